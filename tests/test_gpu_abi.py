"""The C ABI on the GPU: argument validation before any enqueue, the sticky
lost state, host-forced fault injection, the device error word for bad ids.
Every failure here is forced from the host: no kernel faults or hangs."""
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


@pytest.fixture(scope="module")
def tiny():
    wl = syn.WORKLOADS["tiny"]
    return wl, syn.make_layer_weights(wl, 0, "cuda")


def _setup(moe, wl, W, rows=2):
    from routed_fp8_expert_amd.workload import layer_weights
    lw = layer_weights(wl, W)
    x = syn.make_x(wl, 0, rows, 0, "cuda")
    y = torch.full((rows, wl.hidden), 7.0, dtype=torch.bfloat16, device="cuda")
    rt = moe.Routing(rows, wl.n_experts, wl.top_k, "cuda")
    rt.topk_ids.fill_(-7)
    ws = moe.workspace(lw, rows, "cuda")
    return lw, x, y, rt, ws


def _untouched(y, rt):
    torch.cuda.synchronize()
    return bool(torch.all(y == 7.0)) and bool(torch.all(rt.topk_ids == -7))


def test_rejections_enqueue_nothing(moe, tiny):
    wl, W = tiny
    ctx = moe.Ctx(0)
    lw, x, y, rt, ws = _setup(moe, wl, W)
    L = moe.binding.lib()
    st = torch.cuda.current_stream().cuda_stream
    H = wl.hidden

    def call(lwc=lw.c, xp=x.data_ptr(), rows=2, ldx=H, yp=y.data_ptr(), ldy=H, wsp=ws.data_ptr(),
             wsn=ws.numel(), routing=rt.ref):
        return L.moe_layer_forward(ctx.handle, C.byref(lwc), xp, rows, ldx, None, routing, yp, None,
                                   ldy, wsp, wsn, st)

    assert call(xp=None) == moe.binding.MOE_ERR_INVALID_ARG
    assert call(xp=x.data_ptr() + 2) == moe.binding.MOE_ERR_MISALIGNED
    assert call(ldx=H - 8) == moe.binding.MOE_ERR_INVALID_ARG
    assert call(ldx=H + 4) == moe.binding.MOE_ERR_MISALIGNED
    assert call(yp=None) == moe.binding.MOE_ERR_INVALID_ARG
    assert call(wsn=16) == moe.binding.MOE_ERR_WORKSPACE_TOO_SMALL
    assert call(wsp=None) == moe.binding.MOE_ERR_INVALID_ARG
    assert call(rows=-1) == moe.binding.MOE_ERR_INVALID_ARG
    assert call(rows=1025) == moe.binding.MOE_ERR_UNSUPPORTED_SHAPE
    bad = moe.binding.LayerWeightsC.from_buffer_copy(lw.c)
    bad.hidden = 200
    assert call(lwc=bad) == moe.binding.MOE_ERR_UNSUPPORTED_SHAPE
    bad = moe.binding.LayerWeightsC.from_buffer_copy(lw.c)
    bad.top_k = 17
    assert call(lwc=bad) == moe.binding.MOE_ERR_UNSUPPORTED_SHAPE
    bad = moe.binding.LayerWeightsC.from_buffer_copy(lw.c)
    bad.routed.gate_up = lw.c.routed.gate_up + 4
    assert call(lwc=bad) == moe.binding.MOE_ERR_MISALIGNED
    bad = moe.binding.LayerWeightsC.from_buffer_copy(lw.c)
    bad.router_w = None
    assert call(lwc=bad) == moe.binding.MOE_ERR_INVALID_ARG
    badr = moe.binding.RoutingC.from_buffer_copy(rt.c)
    badr.perm = None
    assert call(routing=C.byref(badr)) == moe.binding.MOE_ERR_INVALID_ARG
    assert _untouched(y, rt)
    assert moe.moe_ctx_status(ctx) == 0
    # and the same ctx still works afterwards
    moe.moe_layer_forward(ctx, lw, x, y, None, ws, routing=rt)
    torch.cuda.synchronize()
    assert not torch.all(y == 7.0)
    ctx.close()


def test_fault_injection_is_sticky(moe, tiny):
    wl, W = tiny
    ctx = moe.Ctx(0)
    lw, x, y, rt, ws = _setup(moe, wl, W, rows=1)
    moe.moe_ctx_set_fault_at(ctx, 1)          # the very first launch fails
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_layer_forward(ctx, lw, x, y, None, ws, routing=rt)
    assert ei.value.status == moe.binding.MOE_ERR_DEVICE_LOST
    assert moe.moe_ctx_status(ctx) == moe.binding.MOE_ERR_DEVICE_LOST
    for _ in range(2):
        with pytest.raises(moe.MoeError) as ei:
            moe.moe_layer_forward(ctx, lw, x, y, None, ws, routing=rt)
        assert ei.value.status == moe.binding.MOE_ERR_DEVICE_LOST
    assert _untouched(y, rt)
    ctx.close()
    fresh = moe.Ctx(0)
    moe.moe_layer_forward(fresh, lw, x, y, None, ws, routing=rt)
    torch.cuda.synchronize()
    assert moe.moe_ctx_status(fresh) == 0 and not torch.all(y == 7.0)
    fresh.close()


def test_fault_mid_layer_stops_later_launches(moe, tiny):
    wl, W = tiny
    ctx = moe.Ctx(0)
    moe.moe_ctx_set_one_row_path(ctx, 1)
    lw, x, y, rt, ws = _setup(moe, wl, W, rows=1)
    # on the three-launch path (router + shared expert, routed gate/up, down +
    # blend) the third launch is refused, the first two have run
    moe.moe_ctx_set_fault_at(ctx, 3)
    with pytest.raises(moe.MoeError):
        moe.moe_layer_forward(ctx, lw, x, y, None, ws, routing=rt)
    torch.cuda.synchronize()
    assert torch.all(y == 7.0)                 # no output written after the fault
    assert not torch.all(rt.topk_ids == -7)   # the launches before it did run
    ctx.close()


def test_bad_ids_are_skipped_and_flagged(moe, tiny):
    wl, W = tiny
    ctx = moe.Ctx(0)
    lw, x, y, rt, ws = _setup(moe, wl, W, rows=1)
    moe.moe_route(ctx, lw, x, rt, ws)
    torch.cuda.synchronize()
    assert moe.moe_ctx_device_errors(ctx) == 0
    rt.topk_ids[0, 0] = wl.n_experts + 5
    moe.moe_expert_ffn(ctx, lw, x, rt, y, None, ws)
    assert moe.moe_ctx_device_errors(ctx) & 1
    assert torch.all(torch.isfinite(y.float()))
    # multi-row, grouped path: a corrupt permutation is caught, not followed
    lw2, x2, y2, rt2, ws2 = _setup(moe, wl, W, rows=4)
    moe.moe_route(ctx, lw2, x2, rt2, ws2)
    rt2.perm.fill_(1 << 20)
    moe.moe_ctx_set_few_rows(ctx, 0)
    moe.moe_expert_ffn(ctx, lw2, x2, rt2, y2, None, ws2)
    assert moe.moe_ctx_device_errors(ctx) & 1
    # multi-row, few-rows path (no grouping read): a bad id is skipped and flagged
    moe.moe_ctx_set_few_rows(ctx, 8)
    moe.moe_route(ctx, lw2, x2, rt2, ws2)
    rt2.topk_ids[2, 1] = -3
    moe.moe_expert_ffn(ctx, lw2, x2, rt2, y2, None, ws2)
    assert moe.moe_ctx_device_errors(ctx) & 1
    assert torch.all(torch.isfinite(y2.float()))
    assert moe.moe_ctx_status(ctx) == 0
    ctx.close()


def test_route_then_ffn_equals_layer_forward(moe, tiny):
    wl, W = tiny
    ctx = moe.Ctx(0)
    for rows in (1, 5):
        lw, x, y, rt, ws = _setup(moe, wl, W, rows=rows)
        moe.moe_layer_forward(ctx, lw, x, y, None, ws, routing=rt)
        y2 = torch.empty_like(y)
        rt2 = moe.Routing(rows, wl.n_experts, wl.top_k, "cuda")
        ws2 = moe.workspace(lw, rows, "cuda")
        moe.moe_route(ctx, lw, x, rt2, ws2)
        moe.moe_expert_ffn(ctx, lw, x, rt2, y2, None, ws2)
        torch.cuda.synchronize()
        assert torch.equal(rt.topk_ids, rt2.topk_ids)
        assert torch.equal(y.view(torch.int16), y2.view(torch.int16))
    ctx.close()


def test_kernel_timing_counts_launches(moe, tiny):
    wl, W = tiny
    ctx = moe.Ctx(0)
    lw, x, y, rt, ws = _setup(moe, wl, W, rows=1)
    layer = moe.KERNELS.index("layer")
    moe.moe_ctx_set_timing(ctx, True)
    for _ in range(3):
        moe.moe_layer_forward(ctx, lw, x, y, None, ws, routing=rt)
    ms, n = moe.moe_ctx_kernel_stats(ctx, layer)
    assert n == 3 and ms > 0
    moe.moe_ctx_set_one_row_path(ctx, 1)
    moe.moe_ctx_set_timing(ctx, True)
    for _ in range(2):
        moe.moe_layer_forward(ctx, lw, x, y, None, ws, routing=rt)
    assert moe.moe_ctx_kernel_stats(ctx, 3)[1] == 2
    assert moe.moe_ctx_kernel_stats(ctx, 0)[1] == 2
    assert moe.moe_ctx_kernel_stats(ctx, layer)[1] == 0
    moe.moe_ctx_set_timing(ctx, False)
    ctx.close()


@pytest.mark.parametrize("name,single", [("a3b", True), ("a17b", False)])
def test_single_launch_only_where_resident(moe, name, single):
    """The one-row layer takes the single launch for the 35B-A3B shape (all
    its workgroups fit on the GPU at once) and the three launches for the
    397B-A17B shape (they do not)."""
    wl = syn.WORKLOADS[name]
    W = syn.make_layer_weights(wl, 0, "cuda")
    ctx = moe.Ctx(0)
    lw, x, y, rt, ws = _setup(moe, wl, W, rows=1)
    moe.moe_ctx_set_timing(ctx, True)
    moe.moe_layer_forward(ctx, lw, x, y, None, ws, routing=rt)
    layer = moe.moe_ctx_kernel_stats(ctx, moe.KERNELS.index("layer"))[1]
    router = moe.moe_ctx_kernel_stats(ctx, moe.KERNELS.index("router"))[1]
    assert (layer, router) == ((1, 0) if single else (0, 1))
    assert moe.moe_ctx_device_errors(ctx) == 0
    moe.moe_ctx_set_timing(ctx, False)
    ctx.close()


def test_fault_injection_on_single_launch_layer(moe, tiny):
    wl, W = tiny
    ctx = moe.Ctx(0)
    lw, x, y, rt, ws = _setup(moe, wl, W, rows=1)
    moe.moe_ctx_set_fault_at(ctx, 2)
    moe.moe_layer_forward(ctx, lw, x, y, None, ws, routing=rt)     # launch 1 runs
    with pytest.raises(moe.MoeError):
        moe.moe_layer_forward(ctx, lw, x, y, None, ws, routing=rt)  # launch 2 refused
    assert moe.moe_ctx_status(ctx) == moe.binding.MOE_ERR_DEVICE_LOST
    ctx.close()


@pytest.mark.parametrize("name", ["tiny", "a3b"])
def test_wait_limit_zero_times_out_and_recovers(moe, orc, name):
    """A wait limit of zero makes every waiting workgroup of the one-launch
    layer give up after a single poll (forced from the host: every kernel
    still exits).  At the 35B-A3B shape the down workgroups' wait for the
    experts' h cannot have been met by then, so bit 1 of the device error
    word is set.  Clearing the word also resets the ctx's synchronisation
    words, and the next call, at the default limit, matches the oracle."""
    from gpu_helpers import check_layer, oracle_threads
    from helpers import tie_free_x
    wl = syn.WORKLOADS[name]
    W = syn.make_layer_weights(wl, 0, "cuda")
    ctx = moe.Ctx(0)
    lw, _, y, rt, ws = _setup(moe, wl, W, rows=1)
    x, _ = tie_free_x(orc, wl, W, 0, 1, device="cuda")
    res0 = syn.make_residual(wl, 0, 1, "cuda")
    moe.moe_ctx_set_timing(ctx, True)
    moe.moe_ctx_set_wait_limit(ctx, 0)
    print(f"wait limit 0: {name}", flush=True)
    for _ in range(3):
        moe.moe_layer_forward(ctx, lw, x, y, res0.clone(), ws, routing=rt)
    torch.cuda.synchronize()
    assert moe.moe_ctx_kernel_stats(ctx, moe.KERNELS.index("layer"))[1] == 3
    flags = moe.moe_ctx_device_errors(ctx, clear=True)
    if name == "a3b":
        assert flags & 2, f"no wait timed out at limit 0 (flags {flags})"
    assert flags & ~3 == 0
    moe.moe_ctx_set_wait_limit(ctx, -1)
    res = res0.clone()
    print(f"default wait limit after clearing: {name}", flush=True)
    moe.moe_layer_forward(ctx, lw, x, y, res, ws, routing=rt)
    torch.cuda.synchronize()
    assert moe.moe_ctx_device_errors(ctx, clear=False) == 0
    orc.set_threads(oracle_threads())
    check_layer(orc, wl, W, x, None, res0, y, res, rt, what=f"{name} after a forced timeout")
    ctx.close()


def test_ctx_pool_slots_are_reused(moe):
    """Ctxs take their synchronisation words from a fixed pool (64 per
    device): ctxs are created until the pool is full (at most 64, fewer if
    other ctxs are alive), the next one is refused with
    MOE_ERR_TOO_MANY_CTX, and destroying one frees its slot."""
    import gc
    gc.collect()
    live = []
    with pytest.raises(moe.MoeError) as ei:
        for _ in range(65):
            live.append(moe.Ctx(0))
    assert ei.value.status == moe.binding.MOE_ERR_TOO_MANY_CTX
    assert 1 <= len(live) <= 64
    live.pop().close()
    extra = moe.Ctx(0)
    for c in live + [extra]:
        c.close()
