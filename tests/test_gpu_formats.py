"""GPU parity of the other expert formats (int8 per row, int4 per row,
int4-g64, fp8 with bf16 block scales) through the C ABI against the oracle on
the same seeded inputs, at
the layer's bar (ids and grouping bit-exact, y within 2e-2 * rms and 5e-3
mean relative error).  They run on the GEMV arm and the three-launch one-row
path; forcing the matrix-core arm leaves them on the GEMV arm, and three rows
in one call give the bits of three one-row calls."""
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


@pytest.fixture(scope="module")
def ctx(moe):
    c = moe.Ctx(0)
    yield c
    c.close()


@pytest.fixture(autouse=True)
def _threads(orc):
    orc.set_threads(oracle_threads())


_W = {}


def _weights(wl, layer):
    key = (wl.name, layer)
    if key not in _W:
        _W.clear()
        _W[key] = syn.make_layer_weights(wl, layer, "cuda")
    return _W[key]


def _forward(moe, ctx, wl, W, x, li, res0):
    from routed_fp8_expert_amd.workload import layer_weights
    R = x.shape[0]
    lw = layer_weights(wl, W)
    rt = moe.Routing(R, wl.n_experts, wl.top_k, "cuda", logits=True)
    ws = moe.workspace(lw, R, "cuda")
    y = torch.full((R, wl.hidden), float("nan"), dtype=torch.bfloat16, device="cuda")
    res = res0.clone()
    moe.moe_layer_forward(ctx, lw, x, y, res, ws, logits_in=li, routing=rt)
    torch.cuda.synchronize()
    return y, res, rt


def _inputs(orc, wl, W, layer, rows):
    """Router-GEMV rows redrawn until tie-free up to 17 rows; beyond, given
    uniform logits (as the multi-row fp8 workload), which need no redraw."""
    res0 = syn.make_residual(wl, layer, rows, "cuda")
    if rows <= 17:
        x, _ = tie_free_x(orc, wl, W, layer, rows, device="cuda")
        return x, syn.make_logits_in(wl, layer, rows, "cuda"), res0
    x = syn.make_x(wl, layer, rows, 0, "cuda")
    return x, syn.make_logits_in(syn.WORKLOADS["a3b_multi"], layer, rows, "cuda"), res0


CASES = [("tiny_i4g64", 0, r) for r in (1, 3, 17)] + \
        [("a3b_i8", 0, 1), ("a3b_i8", 1, 8), ("a3b_i8", 0, 33)] + \
        [("a3b_i4", 0, 1), ("a3b_i4", 0, 8)] + \
        [("a3b_i4g64", 0, 1), ("a3b_i4g64", 1, 1), ("a3b_i4g64", 0, 8), ("a3b_i4g64", 0, 64)] + \
        [("tiny_f8bs", 0, 1), ("tiny_f8bs", 0, 5), ("a3b_f8bs", 0, 1), ("a3b_f8bs", 0, 8), ("a3b_f8bs", 0, 64)]


@pytest.mark.parametrize("name,layer,rows", CASES)
def test_int_format_layer(moe, ctx, orc, name, layer, rows):
    wl = syn.WORKLOADS[name]
    W = _weights(wl, layer)
    x, li, res0 = _inputs(orc, wl, W, layer, rows)
    print(f"{name}: layer {layer}, rows {rows}", flush=True)
    y, res, rt = _forward(moe, ctx, wl, W, x, li, res0)
    assert moe.moe_ctx_status(ctx) == 0
    sample = None if rows <= 17 else [0, 1, rows // 2, rows - 1]
    stats = check_layer(orc, wl, W, x, li, res0, y, res, rt, rows=sample, what=f"{name} L{layer} R{rows}")
    print(f"  max|err|/rms {stats[0]:.2e}, mean rel {stats[1]:.2e}", flush=True)


@pytest.mark.parametrize("name", ["a3b_i8", "a3b_i4g64", "a3b_f8bs"])
def test_int_formats_stay_on_gemv_arm_and_one_row_paths_agree(moe, orc, name):
    wl = syn.WORKLOADS[name]
    W = _weights(wl, 0)
    x, li, res0 = _inputs(orc, wl, W, 0, 8)
    print(f"{name}: forced arms, 8 rows; one-row paths", flush=True)
    outs = []
    for arm in (0, 1, 2):        # default, GEMV forced, matrix cores forced
        c = moe.Ctx(0)
        moe.moe_ctx_set_force_arm(c, arm)
        y, res, _ = _forward(moe, c, wl, W, x, li, res0)
        assert moe.moe_ctx_status(c) == 0
        c.close()
        outs.append(bits(y))
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])
    one = []
    for path in (0, 1):
        c = moe.Ctx(0)
        moe.moe_ctx_set_one_row_path(c, path)
        y, _, _ = _forward(moe, c, wl, W, x[:1], li[:1] if li is not None else None, res0[:1])
        c.close()
        one.append(bits(y))
    assert np.array_equal(one[0], one[1])


@pytest.mark.parametrize("name", ["a3b_i8", "a3b_i4", "a3b_i4g64", "a3b_f8bs"])
def test_int_format_batch_invariance(moe, ctx, orc, name):
    """Three rows in one call give the bits of three one-row calls."""
    wl = syn.WORKLOADS[name]
    W = _weights(wl, 0)
    x, li, res0 = _inputs(orc, wl, W, 0, 3)
    print(f"{name}: batch invariance", flush=True)
    y3, _, _ = _forward(moe, ctx, wl, W, x, li, res0)
    for r in range(3):
        y1, _, _ = _forward(moe, ctx, wl, W, x[r:r + 1], None if li is None else li[r:r + 1], res0[r:r + 1])
        assert np.array_equal(bits(y3[r:r + 1]), bits(y1)), f"row {r}"
