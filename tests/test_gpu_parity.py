"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs, for every workload, plus the kernels' own format
converters, determinism and batch invariance."""
import numpy as np
import pytest
import torch

import moe_synth as syn
from gpu_helpers import check_layer, make_tie_free, need_gpu, oracle_threads
from helpers import bits, host, tie_free_x

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


def _say(msg):
    print(msg, flush=True)


# ------------------------------------------------------------------ formats

def test_decode_probe_e4m3(moe, ctx, orc):
    codes = torch.arange(256, dtype=torch.uint8, device="cuda")
    out = torch.empty(512, dtype=torch.float32, device="cuda")
    moe.moe_debug_decode(ctx, 0, codes, out)
    torch.cuda.synchronize()
    o = out.cpu().numpy().reshape(256, 2)
    ref = orc.e4m3_to_f32(np.arange(256, dtype=np.uint8))
    ok = ~np.isnan(ref)
    for path in range(2):
        assert np.array_equal(o[ok, path].view(np.uint32), ref[ok].view(np.uint32)), f"path {path}"


def test_decode_probe_e2m1(moe, ctx, orc):
    codes = torch.arange(256, dtype=torch.uint8, device="cuda")
    out = torch.empty(1024, dtype=torch.float32, device="cuda")
    moe.moe_debug_decode(ctx, 1, codes, out)
    torch.cuda.synchronize()
    o = out.cpu().numpy().reshape(256, 4)
    b = np.arange(256, dtype=np.uint8)
    lo, hi = orc.e2m1_to_f32(b & 15), orc.e2m1_to_f32(b >> 4)
    for path in (0, 2):
        assert np.array_equal(o[:, path], lo), f"low nibble path {path}"
        assert np.array_equal(o[:, path + 1], hi), f"high nibble path {path}"


# ------------------------------------------------------------------ helpers

def _run(moe, ctx, wl, W, x, logits_in=None, residual0=None, rows_routing=True, layer=0):
    from routed_fp8_expert_amd.workload import layer_weights
    R = x.shape[0]
    lw = layer_weights(wl, W)
    rt = moe.Routing(R, wl.n_experts, wl.top_k, "cuda", logits=True)
    ws = moe.workspace(lw, R, "cuda")
    y = torch.full((R, wl.hidden), float("nan"), dtype=torch.bfloat16, device="cuda")
    if residual0 is None:
        residual0 = syn.make_residual(wl, layer, R, "cuda")
    res = residual0.clone()
    moe.moe_layer_forward(ctx, lw, x, y, res, ws, logits_in=logits_in, routing=rt)
    torch.cuda.synchronize()
    return y, res, rt, residual0


def _layer(moe, ctx, orc, wl, layer, rows, sample_rows=None, W=None):
    W = W if W is not None else syn.make_layer_weights(wl, layer, "cuda")
    if wl.router == "gemv":
        x, _ = tie_free_x(orc, wl, W, layer, rows, device="cuda")
    else:
        x = syn.make_x(wl, layer, rows, 0, "cuda")
    li = syn.make_logits_in(wl, layer, rows, "cuda")
    _say(f"{wl.name}: layer {layer}, rows {rows}")
    y, res, rt, res0 = _run(moe, ctx, wl, W, x, li, layer=layer)
    assert moe.moe_ctx_status(ctx) == 0
    stats = check_layer(orc, wl, W, x, li, res0, y, res, rt, rows=sample_rows,
                        what=f"{wl.name} L{layer} R{rows}")
    _say(f"  max|err|/rms {stats[0]:.2e}, mean rel {stats[1]:.2e}")
    return stats


# ------------------------------------------------------------------ workloads

def test_tiny_one_row(moe, ctx, orc):
    _layer(moe, ctx, orc, syn.WORKLOADS["tiny"], 0, 1)


@pytest.mark.parametrize("rows", [2, 3, 5, 17, 64])
def test_tiny_multi_row_gemv_router(moe, ctx, orc, rows):
    _layer(moe, ctx, orc, syn.WORKLOADS["tiny"], 0, rows)


@pytest.mark.parametrize("layer", [0, 1, 39])
def test_a3b_one_row(moe, ctx, orc, layer):
    _layer(moe, ctx, orc, syn.WORKLOADS["a3b"], layer, 1)


# 9 rows: the first grouped step with the matrix-core arm (8 and fewer take
# the few-rows path)
@pytest.mark.parametrize("rows", [2, 4, 8, 9, 12, 16, 32, 64])
def test_a3b_multi_row(moe, ctx, orc, rows):
    wl = syn.WORKLOADS["a3b_multi"]
    for layer in (0, 1):
        _layer(moe, ctx, orc, wl, layer, rows)


@pytest.mark.parametrize("rows", [1, 8])
def test_a17b_nvfp4(moe, ctx, orc, rows):
    _layer(moe, ctx, orc, syn.WORKLOADS["a17b"], 0, rows)


def test_a3b_zipf_64(moe, ctx, orc):
    _layer(moe, ctx, orc, syn.WORKLOADS["a3b_zipf"], 0, 64)


def test_a3b_zipf_512_sampled(moe, ctx, orc):
    wl = syn.WORKLOADS["a3b_zipf"]
    li = syn.make_logits_in(wl, 0, 512, "cpu")
    ids = li.topk(wl.top_k, dim=1).indices
    hot = int(torch.bincount(ids.flatten(), minlength=wl.n_experts).argmax())
    hot_rows = torch.where((ids == hot).any(1))[0][:8].tolist()
    sample = sorted(set(hot_rows + [0, 1, 255, 256, 510, 511] + list(range(100, 108))))
    _layer(moe, ctx, orc, wl, 0, 512, sample_rows=sample)


def test_a3b_forty_layers_as_benchmarked(moe, ctx, orc):
    """The benchmark's configuration: 40 resident layers, one row, run back to
    back on one stream; every layer checked."""
    from routed_fp8_expert_amd.workload import Resident
    wl = syn.WORKLOADS["a3b"]
    _say("a3b: building 40 resident layers")
    res = Resident(wl, 1, device="cuda")
    make_tie_free(orc, res)
    res.run(ctx)
    torch.cuda.synchronize()
    assert moe.moe_ctx_status(ctx) == 0
    worst = 0.0
    for n, l in enumerate(res.layer_ids):
        st = check_layer(orc, wl, res.W[n], res.x[n], None, res.residual0[n], res.y[n],
                         res.residual[n], res.routing[n], what=f"a3b L{l}")
        worst = max(worst, st[0])
    assert moe.moe_ctx_device_errors(ctx) == 0
    _say(f"  40 layers ok, worst max|err|/rms {worst:.2e}")


# ------------------------------------------------------------------ variants

def _tiny_with(**changes):
    wl = syn.WORKLOADS["tiny"]
    W = syn.make_layer_weights(wl, 0, "cuda")
    for k, v in changes.items():
        W[k] = v
    return wl, W


def test_no_residual_no_bias_ungated_shared(moe, ctx, orc):
    import dataclasses
    wl, W = _tiny_with(router_bias=None, shared_gate_w=None)
    x, _ = tie_free_x(orc, wl, W, 0, 3, device="cuda")
    y, res, rt, res0 = _run(moe, ctx, wl, W, x)
    assert torch.all(rt.shared_gate == 1.0)
    check_layer(orc, wl, W, x, None, res0, y, res, rt, what="ungated")


def test_without_shared_expert(moe, ctx, orc):
    import dataclasses
    wl0 = syn.WORKLOADS["tiny"]
    wl = dataclasses.replace(wl0, shared_inter=0)
    W = syn.make_layer_weights(wl, 0, "cuda")
    x, _ = tie_free_x(orc, wl, W, 0, 2, device="cuda")
    y, res, rt, res0 = _run(moe, ctx, wl, W, x)
    check_layer(orc, wl, W, x, None, res0, y, res, rt, what="no shared")


@pytest.mark.parametrize("k", [1, 16])
def test_top_k_extremes(moe, ctx, orc, k):
    import dataclasses
    wl = dataclasses.replace(syn.WORKLOADS["tiny"], top_k=k)
    W = syn.make_layer_weights(wl, 0, "cuda")
    x, _ = tie_free_x(orc, wl, W, 0, 4, device="cuda")
    y, res, rt, res0 = _run(moe, ctx, wl, W, x)
    check_layer(orc, wl, W, x, None, res0, y, res, rt, what=f"k={k}")
    if k == 1:
        assert torch.all(rt.topk_w == 1.0)


ODD_SHAPES = {
    # hidden 3 K blocks, 100 experts (not a multiple of the wave), shared
    # intermediate half the routed one
    "h384_e100": dict(hidden=384, n_experts=100, top_k=6, inter=256, shared_inter=128),
    # hidden 9 K blocks (odd), 200 experts, shared intermediate three times the
    # routed one (3 K blocks in its down projection)
    "h1152_e200": dict(hidden=1152, n_experts=200, top_k=3, inter=128, shared_inter=384),
}


ODD_CASES = [(shape, 0) for shape in ODD_SHAPES] + [("h384_e100", f) for f in (1, 2, 3, 4, 5)]


@pytest.mark.parametrize("shape,fmt", ODD_CASES)
@pytest.mark.parametrize("rows", [1, 5, 40])
def test_odd_shapes(moe, ctx, orc, shape, fmt, rows):
    """Shapes away from the models': expert counts that do not fill the top-k
    lanes, shared and routed intermediates that differ, odd K-block counts;
    one row (three-launch path), a few rows and a matrix-core step (fp8), in
    every weight format."""
    import dataclasses
    wl = dataclasses.replace(syn.WORKLOADS["tiny"], name=f"odd_{shape}", fmt=fmt, **ODD_SHAPES[shape])
    W = syn.make_layer_weights(wl, 0, "cuda")
    li = None
    if rows <= 8:
        x, _ = tie_free_x(orc, wl, W, 0, rows, device="cuda")
    else:
        # many rows of 100+ experts: given logits (compared as the same f32
        # values on both sides), the router GEMV skipped
        x = syn.make_x(wl, 0, rows, 0, "cuda")
        li = syn.make_logits_in(dataclasses.replace(wl, router="uniform"), 0, rows, "cuda")
    _say(f"{wl.name}: rows {rows}")
    y, res, rt, res0 = _run(moe, ctx, wl, W, x, li)
    assert moe.moe_ctx_status(ctx) == 0 and moe.moe_ctx_device_errors(ctx) == 0
    check_layer(orc, wl, W, x, li, res0, y, res, rt, what=f"{shape} fmt {fmt} R{rows}")


def test_padded_leading_dimensions(moe, ctx, orc):
    from routed_fp8_expert_amd.workload import layer_weights
    wl = syn.WORKLOADS["tiny"]
    W = syn.make_layer_weights(wl, 0, "cuda")
    x, _ = tie_free_x(orc, wl, W, 0, 3, device="cuda")
    xp = torch.zeros((3, wl.hidden + 64), dtype=torch.bfloat16, device="cuda")
    xp[:, : wl.hidden] = x
    res0 = syn.make_residual(wl, 0, 3, "cuda")
    yp = torch.zeros((3, wl.hidden + 32), dtype=torch.bfloat16, device="cuda")
    rp = torch.zeros((3, wl.hidden + 32), dtype=torch.bfloat16, device="cuda")
    rp[:, : wl.hidden] = res0
    lw = layer_weights(wl, W)
    rt = moe.Routing(3, wl.n_experts, wl.top_k, "cuda")
    ws = moe.workspace(lw, 3, "cuda")
    moe.moe_layer_forward(ctx, lw, xp[:, : wl.hidden], yp[:, : wl.hidden], rp[:, : wl.hidden], ws,
                          routing=rt)
    torch.cuda.synchronize()
    assert torch.all(yp[:, wl.hidden:] == 0) and torch.all(rp[:, wl.hidden:] == 0)
    check_layer(orc, wl, W, x, None, res0, yp[:, : wl.hidden], rp[:, : wl.hidden], rt, what="padded")


def test_zero_rows_is_a_no_op(moe, ctx):
    from routed_fp8_expert_amd.workload import layer_weights
    wl = syn.WORKLOADS["tiny"]
    W = syn.make_layer_weights(wl, 0, "cuda")
    lw = layer_weights(wl, W)
    x = torch.empty((0, wl.hidden), dtype=torch.bfloat16, device="cuda")
    y = torch.empty((0, wl.hidden), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(256, dtype=torch.uint8, device="cuda")
    moe.moe_layer_forward(ctx, lw, x, y, None, ws)
    torch.cuda.synchronize()
    assert moe.moe_ctx_status(ctx) == 0


def test_max_rows_with_given_logits(moe, ctx, orc):
    wl = syn.WORKLOADS["a3b_multi"]
    _layer(moe, ctx, orc, wl, 0, 1024, sample_rows=[0, 1, 511, 512, 1022, 1023])


# ------------------------------------------------------------------ arms

@pytest.mark.parametrize("rows", [2, 5, 33, 64])
def test_mfma_arm_forced_for_every_expert(moe, ctx, orc, rows):
    """Every expert with at least one row (and the shared expert) on the
    matrix-core arm, including tiles with a single valid row."""
    moe.moe_ctx_set_force_arm(ctx, 2)
    try:
        _layer(moe, ctx, orc, syn.WORKLOADS["a3b_multi"], 2, rows)
        assert moe.moe_ctx_device_errors(ctx) == 0
    finally:
        moe.moe_ctx_set_force_arm(ctx, 0)


def _logits_with_counts(E, k, R, counts, seed):
    """Given router logits under which expert e (a key of `counts`) is chosen
    by exactly counts[e] rows: each listed expert takes the rows with the
    fewest choices so far, every row is then filled to k distinct experts
    from the unlisted ones in turn (1-3 rows each), and a row's chosen
    experts get distinct logits well above all others (tie-free)."""
    rng = np.random.default_rng(seed)
    chosen = [[] for _ in range(R)]
    for e, c in counts.items():
        load = np.array([len(ch) for ch in chosen])
        for r in np.argsort(load, kind="stable")[:c]:
            chosen[r].append(e)
    fill = [e for e in range(E) if e not in counts]
    nxt = 0
    for r in range(R):
        assert len(chosen[r]) <= k
        while len(chosen[r]) < k:
            e = fill[nxt % len(fill)]
            nxt += 1
            if e not in chosen[r]:
                chosen[r].append(e)
    li = rng.normal(0.0, 1.0, size=(R, E)).astype(np.float32)
    for r in range(R):
        top = 10.0 + rng.permutation(k).astype(np.float32) * 0.37 + rng.uniform(0, 0.1, k).astype(np.float32)
        li[r, chosen[r]] = top
    return li


@pytest.mark.parametrize("rows,counts", [
    (160, {3: 4, 7: 16, 9: 17, 11: 31, 12: 32, 13: 33, 20: 48, 21: 63, 22: 64, 23: 65, 30: 100, 31: 129,
           40: 160}),
    (512, {0: 512, 1: 300, 2: 257, 3: 129, 4: 64, 5: 63, 6: 16, 7: 4}),
])
def test_mfma_tile_shapes(moe, ctx, orc, rows, counts):
    """Experts whose row counts give gate/up tiles of 1 to 4 16-row subtiles
    (ragged last subtiles, several tiles per expert, an expert on every row)
    and down tiles with ragged tails, against the oracle."""
    wl = syn.WORKLOADS["a3b_multi"]
    W = syn.make_layer_weights(wl, 6, "cuda")
    x = syn.make_x(wl, 6, rows, 0, "cuda")
    li = torch.from_numpy(_logits_with_counts(wl.n_experts, wl.top_k, rows, counts, 60 + rows)).cuda()
    _say(f"{wl.name}: given counts, rows {rows}")
    y, res, rt, res0 = _run(moe, ctx, wl, W, x, li, layer=6)
    assert moe.moe_ctx_status(ctx) == 0 and moe.moe_ctx_device_errors(ctx) == 0
    got = rt.expert_count.cpu().numpy()
    for e, c in counts.items():
        assert got[e] == c, (e, got[e], c)
    sample = None if rows <= 160 else list(range(0, rows, 37)) + [rows - 1]
    check_layer(orc, wl, W, x, li, res0, y, res, rt, rows=sample, what=f"counts R{rows}")


def test_down_tile_heights_agree(moe, ctx):
    """Steps of 512 rows and more run the matrix-core down projection on
    64-row tiles (a launch of its own), smaller steps on 16-row tiles inside
    the grouped launch: with every expert on the matrix-core arm, the first
    300 rows of a 600-row step give the bits of a 300-row step."""
    wl = syn.WORKLOADS["a3b_zipf"]
    W = syn.make_layer_weights(wl, 7, "cuda")
    x = syn.make_x(wl, 7, 600, 0, "cuda")
    li = syn.make_logits_in(wl, 7, 600, "cuda")
    r0 = syn.make_residual(wl, 7, 600, "cuda")
    moe.moe_ctx_set_force_arm(ctx, 2)
    try:
        _say("a3b_zipf: 600 rows against their first 300, every expert on the matrix cores")
        y6, res6, rt6, _ = _run(moe, ctx, wl, W, x, li, r0)
        y3, res3, rt3, _ = _run(moe, ctx, wl, W, x[:300].contiguous(), li[:300].contiguous(), r0[:300].contiguous())
    finally:
        moe.moe_ctx_set_force_arm(ctx, 0)
    assert moe.moe_ctx_device_errors(ctx) == 0
    assert torch.equal(rt6.topk_ids[:300], rt3.topk_ids)
    assert torch.equal(y6[:300].view(torch.int16), y3.view(torch.int16))
    assert torch.equal(res6[:300].view(torch.int16), res3.view(torch.int16))


def test_gemv_arm_only_at_64_rows(moe, ctx, orc):
    moe.moe_ctx_set_force_arm(ctx, 1)
    try:
        _layer(moe, ctx, orc, syn.WORKLOADS["a3b_zipf"], 3, 64)
    finally:
        moe.moe_ctx_set_force_arm(ctx, 0)


def test_mfma_threshold_one_and_large(moe, ctx, orc):
    wl = syn.WORKLOADS["a3b_zipf"]
    for thr in (1, 40):
        moe.moe_ctx_set_mfma_min_rows(ctx, thr)
        try:
            _layer(moe, ctx, orc, wl, 4, 64)
        finally:
            moe.moe_ctx_set_mfma_min_rows(ctx, 0)


def test_determinism_with_mfma_arm(moe, ctx, orc):
    wl = syn.WORKLOADS["a3b_zipf"]
    W = syn.make_layer_weights(wl, 5, "cuda")
    x = syn.make_x(wl, 5, 64, 0, "cuda")
    li = syn.make_logits_in(wl, 5, 64, "cuda")
    r0 = syn.make_residual(wl, 5, 64, "cuda")
    a = _run(moe, ctx, wl, W, x, li, r0)
    b = _run(moe, ctx, wl, W, x, li, r0)
    assert torch.equal(a[0].view(torch.int16), b[0].view(torch.int16))
    assert moe.moe_ctx_device_errors(ctx) == 0


# ------------------------------------------------------------------ one-row paths

@pytest.mark.parametrize("name,layer", [("tiny", 0), ("a3b", 3), ("a17b", 1)])
def test_one_row_paths_agree(moe, orc, name, layer):
    """The single-launch layer and the three-launch path give the same bits,
    both match the oracle, and no bounded wait timed out."""
    wl = syn.WORKLOADS[name]
    W = syn.make_layer_weights(wl, layer, "cuda")
    x, _ = tie_free_x(orc, wl, W, layer, 1, device="cuda")
    r0 = syn.make_residual(wl, layer, 1, "cuda")
    out = []
    for path in (0, 1):
        c = moe.Ctx(0)
        moe.moe_ctx_set_one_row_path(c, path)
        res = []
        for _ in range(3):   # repeated calls reuse the ctx's synchronisation words
            res.append(_run(moe, c, wl, W, x, None, r0))
        assert moe.moe_ctx_device_errors(c) == 0
        c.close()
        for a in res[1:]:
            assert torch.equal(a[0].view(torch.int16), res[0][0].view(torch.int16))
        out.append(res[0])
    (y0, o0, rt0, _), (y1, o1, rt1, _) = out
    assert torch.equal(rt0.topk_ids, rt1.topk_ids) and torch.equal(rt0.topk_w, rt1.topk_w)
    assert torch.equal(rt0.shared_gate, rt1.shared_gate)
    assert torch.equal(y0.view(torch.int16), y1.view(torch.int16))
    assert torch.equal(o0.view(torch.int16), o1.view(torch.int16))
    check_layer(orc, wl, W, x, None, r0, y0, o0, rt0, what=f"{name} single launch")


def test_one_row_with_given_logits(moe, ctx, orc):
    wl = syn.WORKLOADS["a3b_multi"]
    W = syn.make_layer_weights(wl, 0, "cuda")
    x = syn.make_x(wl, 0, 1, 0, "cuda")
    li = syn.make_logits_in(wl, 0, 1, "cuda")
    y, res, rt, r0 = _run(moe, ctx, wl, W, x, li)
    check_layer(orc, wl, W, x, li, r0, y, res, rt, what="one row, given logits")


# ------------------------------------------------------------------ properties

def test_determinism(moe, ctx, orc):
    wl = syn.WORKLOADS["a3b_multi"]
    W = syn.make_layer_weights(wl, 0, "cuda")
    x = syn.make_x(wl, 0, 16, 0, "cuda")
    li = syn.make_logits_in(wl, 0, 16, "cuda")
    r0 = syn.make_residual(wl, 0, 16, "cuda")
    a = _run(moe, ctx, wl, W, x, li, r0)
    b = _run(moe, ctx, wl, W, x, li, r0)
    assert torch.equal(a[0].view(torch.int16), b[0].view(torch.int16))
    assert torch.equal(a[1].view(torch.int16), b[1].view(torch.int16))
    assert torch.equal(a[2].topk_ids, b[2].topk_ids) and torch.equal(a[2].perm, b[2].perm)


def test_batch_invariance_gemv_arm(moe, ctx, orc):
    """Three rows in one call give the bits of three one-row calls (the
    colibri pull request's decode GEMV convention)."""
    wl = syn.WORKLOADS["a3b"]
    W = syn.make_layer_weights(wl, 2, "cuda")
    x, _ = tie_free_x(orc, wl, W, 2, 3, device="cuda")
    r0 = syn.make_residual(wl, 2, 3, "cuda")
    moe.moe_ctx_set_force_arm(ctx, 1)
    try:
        y3, res3, rt3, _ = _run(moe, ctx, wl, W, x, None, r0)
        for r in range(3):
            y1, res1, rt1, _ = _run(moe, ctx, wl, W, x[r:r + 1].contiguous(), None,
                                    r0[r:r + 1].contiguous())
            assert torch.equal(rt1.topk_ids[0], rt3.topk_ids[r])
            assert torch.equal(rt1.topk_w[0], rt3.topk_w[r])
            assert torch.equal(y1[0].view(torch.int16), y3[r].view(torch.int16)), f"row {r}"
            assert torch.equal(res1[0].view(torch.int16), res3[r].view(torch.int16)), f"row {r}"
    finally:
        moe.moe_ctx_set_force_arm(ctx, 0)
