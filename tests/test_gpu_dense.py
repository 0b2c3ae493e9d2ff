"""GPU tests of the dense fp8 block-128 projection (moe_dense_fp8) through the
C ABI, against the oracle's dense_fp8 on the same seeded inputs.

Bar (f32 accumulation, one bf16 rounding): every output within
2^-8 |y| + 2^-14 sum_k |x_k W_nk| of the oracle's exact f64 value (the first
term covers the bf16 rounding, the second the f32 sums of up to 8192 terms),
and at least 95 % of the outputs bit-equal to the oracle value rounded to
bf16.  Both arms (GEMV below 8 rows, matrix cores from 8) at ragged row
counts on both sides of the switch and every K tier of each arm; rows are
batch-invariant within an arm (rows 1 to 7 give one-row bits); strided
operands; rejected arguments enqueue nothing.
"""
import ctypes as C

import numpy as np
import pytest
import torch

import moe_synth as syn
from gpu_helpers import need_gpu, oracle_threads
from helpers import bits, host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def moe():
    need_gpu()
    import routed_fp8_expert_amd as m
    return m


_cache = {}


def _weights(name):
    if name not in _cache:
        n, k = syn.DENSE_SHAPES[name]
        q, s = syn.make_dense_weights(name, n, k, "cuda")
        _cache[name] = (q, s)
    return _cache[name]


def _run(moe, ctx, w, x, y=None):
    if y is None:
        y = torch.full((x.shape[0], w.n), float("nan"), dtype=torch.bfloat16, device="cuda")
    moe.moe_dense_fp8(ctx, w, x, y)
    torch.cuda.synchronize()
    return y


def _check(orc, q, s, x, y, sel):
    orc.set_threads(oracle_threads())
    qh, sh, xb = host(q), host(s), bits(x)[sel]
    want = orc.dense_fp8(qh, sh, xb)
    absdot = orc.dense_fp8(qh & np.uint8(0x7F), sh, xb & np.uint16(0x7FFF))
    got = orc.bf16_to_f32(bits(y)[sel]).astype(np.float64)
    err = np.abs(got - want)
    bound = 2.0 ** -8 * np.abs(want) + 2.0 ** -14 * absdot
    assert np.all(err <= bound), f"max err {err.max():.3g}, worst excess {(err - bound).max():.3g}"
    same = orc.bf16_to_f32(orc.f32_to_bf16(want.astype(np.float32))) == got
    assert same.mean() >= 0.95, f"only {same.mean():.3f} of the outputs round like the oracle"


CASES = [
    # 129 and 300 rows: several row groups, the last one ragged; 400 rows:
    # 32-column workgroups, groups of two tiles, padding blocks in the grid
    ("small_384x640", r) for r in (1, 3, 7, 8, 17, 33, 64, 128, 129, 300, 400)
] + [
    ("up_4096x2048", r) for r in (1, 5, 7, 8, 31, 64, 128, 200)
] + [
    ("down_2048x4096", r) for r in (1, 7, 8, 32, 128)
] + [
    ("wide_256x8192", r) for r in (1, 5, 8, 40)
]


@pytest.mark.parametrize("name,rows", CASES)
def test_dense_parity(moe, orc, name, rows):
    print(f"dense: {name} rows {rows}", flush=True)
    q, s = _weights(name)
    n, k = q.shape
    x = syn.make_dense_x(name, rows, k, "cuda")
    ctx = moe.Ctx(0)
    y = _run(moe, ctx, moe.DenseWeights(q, s), x)
    assert moe.moe_ctx_status(ctx) == 0
    ctx.close()
    sel = np.arange(rows) if rows * n * k <= (1 << 28) else np.unique([0, 1, rows // 2, rows - 2, rows - 1])
    _check(orc, q, s, x, y, sel)


@pytest.mark.parametrize("name", ["small_384x640", "up_4096x2048", "down_2048x4096"])
def test_dense_batch_invariance(moe, name):
    """Within an arm a row's bits do not depend on the call's other rows: one
    to seven rows (GEMV) agree with one-row calls, and matrix-core calls of
    any row count agree with each other."""
    print(f"dense batch invariance: {name}", flush=True)
    q, s = _weights(name)
    w = moe.DenseWeights(q, s)
    x = syn.make_dense_x(name, 130, q.shape[1], "cuda")
    ctx = moe.Ctx(0)
    y7 = _run(moe, ctx, w, x[:7])
    ones = [_run(moe, ctx, w, x[i:i + 1]) for i in range(7)]
    y3 = _run(moe, ctx, w, x[2:5])
    y8 = _run(moe, ctx, w, x[:8])
    y130 = _run(moe, ctx, w, x)
    y64 = _run(moe, ctx, w, x[64:128])
    y45 = _run(moe, ctx, w, x[85:130])
    y17 = _run(moe, ctx, w, x[100:117])
    ctx.close()
    v = lambda t: t.view(torch.int16)
    for i in range(7):
        assert torch.equal(v(y7[i:i + 1]), v(ones[i])), f"row {i}: seven-row call differs from one-row call"
    assert torch.equal(v(y7[2:5]), v(y3))
    assert torch.equal(v(y130[:8]), v(y8))
    assert torch.equal(v(y130[64:128]), v(y64))
    assert torch.equal(v(y130[85:130]), v(y45))
    assert torch.equal(v(y130[100:117]), v(y17))


@pytest.mark.parametrize("rows", [7, 48])
def test_dense_strided_operands(moe, rows):
    """Row strides beyond the widths (ldx > k, ldy > n, ldw > k) give the
    same bits as packed operands and leave the padding alone."""
    name = "small_384x640"
    q, s = _weights(name)
    n, k = q.shape
    x = syn.make_dense_x(name, rows, k, "cuda")
    ctx = moe.Ctx(0)
    y = _run(moe, ctx, moe.DenseWeights(q, s), x)
    qpad = torch.zeros((n, k + 48), dtype=torch.uint8, device="cuda")
    qpad[:, :k] = q
    xpad = torch.zeros((rows, k + 24), dtype=torch.bfloat16, device="cuda")
    xpad[:, :k] = x
    ypad = torch.full((rows, n + 40), 3.0, dtype=torch.bfloat16, device="cuda")
    moe.moe_dense_fp8(ctx, moe.DenseWeights(qpad[:, :k], s), xpad[:, :k], ypad[:, :n])
    torch.cuda.synchronize()
    ctx.close()
    assert torch.equal(ypad[:, :n].view(torch.int16), y.view(torch.int16))
    assert bool(torch.all(ypad[:, n:] == 3.0))


def test_dense_rejections_enqueue_nothing(moe):
    from routed_fp8_expert_amd.binding import DenseWeightsC, lib, _p, _stream
    name = "small_384x640"
    q, s = _weights(name)
    n, k = q.shape
    x = syn.make_dense_x(name, 4, k, "cuda")
    y = torch.full((4, n), 7.0, dtype=torch.bfloat16, device="cuda")
    ctx = moe.Ctx(0)
    sz = C.sizeof(DenseWeightsC)
    good = DenseWeightsC(sz, _p(q), k, _p(s), n, k)
    bad_w = [
        DenseWeightsC(8, _p(q), k, _p(s), n, k),               # struct too small
        DenseWeightsC(sz, None, k, _p(s), n, k),               # no codes
        DenseWeightsC(sz, _p(q), k, None, n, k),               # no scales
        DenseWeightsC(sz, _p(q), k, _p(s), n - 64, k),         # n not a multiple of 128
        DenseWeightsC(sz, _p(q), k, _p(s), n, k + 64),         # k not a multiple of 128
        DenseWeightsC(sz, _p(q), 8192 + 128, _p(s), n, 8192 + 128),   # k too large
        DenseWeightsC(sz, _p(q), k - 16, _p(s), n, k),         # ldw < k
        DenseWeightsC(sz, _p(q), k + 8, _p(s), n, k),          # ldw not a multiple of 16
        DenseWeightsC(sz, _p(q) + 8, k, _p(s), n, k),          # misaligned codes
        DenseWeightsC(sz, _p(q), k, _p(s) + 2, n, k),          # misaligned scales
        DenseWeightsC(sz, _p(q), k, _p(s), 0, k),              # empty n
    ]
    for w in bad_w:
        assert lib().moe_dense_fp8(ctx.handle, C.byref(w), _p(x), 4, k, _p(y), n, _stream(None)) != 0
    bad_calls = [
        (None, 4, k, _p(y), n),          # no x
        (_p(x), 4, k, None, n),          # no y
        (_p(x), -1, k, _p(y), n),        # negative rows
        (_p(x), 4, k - 8, _p(y), n),     # ldx < k
        (_p(x), 4, k, _p(y), n - 1),     # ldy < n
        (_p(x) + 2, 4, k, _p(y), n),     # misaligned x
        (_p(x), 4, k + 4, _p(y), n),     # ldx not a multiple of 8
        (_p(x), 4, k, _p(y) + 1, n),     # misaligned y
    ]
    for xp, r, ldx, yp, ldy in bad_calls:
        assert lib().moe_dense_fp8(ctx.handle, C.byref(good), xp, r, ldx, yp, ldy, _stream(None)) != 0
    # zero rows: accepted, nothing enqueued
    assert lib().moe_dense_fp8(ctx.handle, C.byref(good), None, 0, k, None, n, _stream(None)) == 0
    torch.cuda.synchronize()
    assert bool(torch.all(y == 7.0))
    assert moe.moe_ctx_status(ctx) == 0
    ctx.close()


def test_dense_kernel_timing(moe):
    name = "small_384x640"
    q, s = _weights(name)
    w = moe.DenseWeights(q, s)
    x = syn.make_dense_x(name, 40, q.shape[1], "cuda")
    ctx = moe.Ctx(0)
    moe.moe_ctx_set_timing(ctx, 1)
    _run(moe, ctx, w, x[:3])
    _run(moe, ctx, w, x)
    ms, launches = moe.moe_ctx_kernel_stats(ctx, moe.KERNELS.index("dense"))
    ctx.close()
    assert launches == 2 and ms > 0
