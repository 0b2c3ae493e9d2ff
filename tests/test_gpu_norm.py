"""GPU tests of the RMSNorm epilogue (moe_layer_forward_norm) through the C
ABI, against the oracle on the same seeded inputs.

- The epilogue leaves the layer's own outputs (y, residual, routing) bit for
  bit as moe_layer_forward writes them.
- The normalised rows agree with the oracle's RMSNorm of the very row bits
  the GPU wrote within one bf16 ulp (f32 against f64 sums of squares can
  round the other way at a tie), and the whole chain (oracle layer, then
  oracle norm) within the layer's bar: max |err| <= 2e-2 * rms + one ulp.
- Every path that carries the epilogue is covered: the one-row single
  launch (its last down workgroup), the three launches (a separate norm
  launch), and the multi-row blend (GEMV and matrix-core arms), fp8 and
  NVFP4, with and without a residual.
"""
import numpy as np
import pytest
import torch

import moe_synth as syn
from gpu_helpers import need_gpu, oracle_threads
from helpers import bits, host, oracle_layer, tie_free_x

pytestmark = pytest.mark.gpu

EPS = 1e-6


@pytest.fixture(scope="module")
def moe():
    need_gpu()
    import routed_fp8_expert_amd as m
    return m


def _gamma(wl, layer):
    rng = np.random.default_rng(syn.subseed("norm-weight", wl.name, layer) % (1 << 32))
    g = 1.0 + 0.1 * rng.standard_normal(wl.hidden)
    return torch.tensor(g, dtype=torch.float32).to(torch.bfloat16).cuda()


def _run(moe, ctx, wl, W, x, li, res0, gamma=None):
    from routed_fp8_expert_amd.workload import layer_weights
    R = x.shape[0]
    lw = layer_weights(wl, W)
    rt = moe.Routing(R, wl.n_experts, wl.top_k, "cuda")
    ws = moe.workspace(lw, R, "cuda")
    y = torch.full((R, wl.hidden), float("nan"), dtype=torch.bfloat16, device="cuda")
    res = res0.clone() if res0 is not None else None
    nout = None
    if gamma is None:
        moe.moe_layer_forward(ctx, lw, x, y, res, ws, logits_in=li, routing=rt)
    else:
        nout = torch.full((R, wl.hidden), float("nan"), dtype=torch.bfloat16, device="cuda")
        moe.moe_layer_forward_norm(ctx, lw, x, y, res, ws, gamma, EPS, nout, logits_in=li, routing=rt)
    torch.cuda.synchronize()
    return y, res, rt, nout


def _ordered(b):
    """bf16 bit patterns as integers in value order (adjacent values differ by 1)."""
    b = b.astype(np.int32)
    return np.where(b & 0x8000, -(b & 0x7FFF), b)


CASES = [
    ("tiny", 1, 0, True),
    ("a3b", 1, 0, True),
    ("a3b", 1, 0, False),
    ("a3b", 1, 1, True),
    ("a3b_multi", 16, 0, True),
    ("a3b_multi", 16, 0, False),
    ("a3b_multi", 64, 0, True),
    ("a17b", 1, 0, True),
]


@pytest.mark.parametrize("name,rows,split,with_res", CASES)
def test_norm_epilogue(moe, orc, name, rows, split, with_res):
    wl = syn.WORKLOADS[name]
    layer = 1
    W = syn.make_layer_weights(wl, layer, "cuda")
    if wl.router == "gemv":
        x, _ = tie_free_x(orc, wl, W, layer, rows, device="cuda")
    else:
        x = syn.make_x(wl, layer, rows, 0, "cuda")
    li = syn.make_logits_in(wl, layer, rows, "cuda")
    res0 = syn.make_residual(wl, layer, rows, "cuda") if with_res else None
    gamma = _gamma(wl, layer)
    print(f"norm epilogue: {name} rows {rows} split {split} residual {with_res}", flush=True)
    ctx = moe.Ctx(0)
    moe.moe_ctx_set_one_row_path(ctx, split)
    y0, r0, rt0, _ = _run(moe, ctx, wl, W, x, li, res0)
    y1, r1, rt1, nout = _run(moe, ctx, wl, W, x, li, res0, gamma)
    assert moe.moe_ctx_device_errors(ctx) == 0
    ctx.close()

    # the epilogue leaves the layer's outputs alone
    assert torch.equal(rt0.topk_ids, rt1.topk_ids)
    assert torch.equal(y0.view(torch.int16), y1.view(torch.int16))
    if with_res:
        assert torch.equal(r0.view(torch.int16), r1.view(torch.int16))

    # the normalised rows: the oracle's RMSNorm of the row the GPU wrote
    src = r1 if with_res else y1
    got = bits(nout)
    want = orc.rms_norm(bits(src), bits(gamma), EPS)
    d = np.abs(_ordered(got) - _ordered(want))
    assert d.max() <= 1, f"{name}: normalised rows off by {d.max()} ulp"
    assert (d > 0).mean() < 0.01

    # the whole chain against the oracle (rows sampled at 64)
    sel = np.arange(rows) if rows <= 16 else np.array([0, rows // 2, rows - 1])
    ids = rt1.topk_ids.cpu().numpy()
    L = oracle_layer(orc, wl, W, experts=np.unique(ids[sel]))
    orc.set_threads(oracle_threads())
    ref = orc.layer_forward(L, bits(x)[sel], logits_in=None if li is None else host(li)[sel],
                            residual=None if res0 is None else bits(res0)[sel])
    want2 = orc.bf16_to_f32(orc.rms_norm(ref["out"], bits(gamma), EPS)).astype(np.float64)
    g = orc.bf16_to_f32(got[sel]).astype(np.float64)
    rms = float(np.sqrt(np.mean(want2 ** 2)))
    ulp = np.abs(want2) * 2.0 ** -7
    assert np.all(np.abs(g - want2) <= 2e-2 * rms + ulp), f"{name}: chain off by {np.abs(g - want2).max():.3g}"


def test_norm_rejections_enqueue_nothing(moe, orc):
    from routed_fp8_expert_amd.binding import NormC, MoeError, lib, _p, _stream
    import ctypes as C
    wl = syn.WORKLOADS["tiny"]
    W = syn.make_layer_weights(wl, 0, "cuda")
    from routed_fp8_expert_amd.workload import layer_weights
    lw = layer_weights(wl, W)
    x = syn.make_x(wl, 0, 1, 0, "cuda")
    y = torch.full((1, wl.hidden), 7.0, dtype=torch.bfloat16, device="cuda")
    ws = moe.workspace(lw, 1, "cuda")
    gamma = _gamma(wl, 0)
    nout = torch.full((1, wl.hidden), 7.0, dtype=torch.bfloat16, device="cuda")
    ctx = moe.Ctx(0)
    H = wl.hidden
    bad = [
        NormC(4, _p(gamma), EPS, _p(nout), H),                       # struct too small
        NormC(C.sizeof(NormC), None, EPS, _p(nout), H),              # no weight
        NormC(C.sizeof(NormC), _p(gamma), EPS, None, H),             # no output
        NormC(C.sizeof(NormC), _p(gamma), -1.0, _p(nout), H),        # negative eps
        NormC(C.sizeof(NormC), _p(gamma), float("nan"), _p(nout), H),
        NormC(C.sizeof(NormC), _p(gamma), float("inf"), _p(nout), H),
        NormC(C.sizeof(NormC), _p(gamma), EPS, _p(nout), H - 1),     # row stride too small
        NormC(C.sizeof(NormC), _p(gamma) + 1, EPS, _p(nout), H),     # misaligned
    ]
    for n in bad:
        rc = lib().moe_layer_forward_norm(ctx.handle, lw.ref, _p(x), 1, H, None, None, _p(y), None, H,
                                          C.byref(n), _p(ws), ws.numel(), _stream(None))
        assert rc != 0
    torch.cuda.synchronize()
    assert bool(torch.all(y == 7.0)) and bool(torch.all(nout == 7.0))
    assert moe.moe_ctx_status(ctx) == 0
    ctx.close()
