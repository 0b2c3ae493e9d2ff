"""Pins of the oracle's integer expert formats (colibri PR: a per-row int4
checkpoint of Qwen3.6, an int4-g64 expert sidecar, int8 rows in its decode
GEMV; layout readings: two's-complement codes, int4 two per byte with the
even column in the low nibble, one f32 scale per row or per 64 consecutive
input columns of a row, multiplying).

Pinned against numpy's own two's-complement views (int8 bytes, int4 by
arithmetic shifts), nibble-order and group-index probes with power-of-two
scales, the equivalences per-row == g64 with equal groups and int8 == int4 on
codes in [-8, 7], identity-selection experts (closed form silu(a x) x), and a
numpy float64 textbook layer over an int4-g64 tiny workload.  A swapped
nibble order, a row/column swap in the scale index, a group size other than
64 or an unsigned reading fails one of them.
"""
import numpy as np
import pytest
import scipy.special
import torch

import moe_synth as syn
from helpers import bits, host, oracle_layer
from test_oracle_layer import _textbook_layer


def _np_int4(nib):
    """Sign-extend nibbles with numpy: shift into the high half of an int8,
    then an arithmetic shift back."""
    n = np.asarray(nib, np.uint8) & np.uint8(15)
    return ((n << np.uint8(4)).view(np.int8) >> 4).astype(np.float32)


def _np_deq_int(fmt, q, s):
    q = np.asarray(q, np.uint8)
    if fmt == syn.FMT_INT8_ROW:
        codes = q.view(np.int8).astype(np.float64)
    else:
        codes = np.empty((q.shape[0], 2 * q.shape[1]), np.float64)
        codes[:, 0::2] = _np_int4(q & 15)
        codes[:, 1::2] = _np_int4(q >> 4)
    G = codes.shape[1] // s.shape[1]
    return (codes * np.repeat(np.asarray(s, np.float64), G, axis=1)).astype(np.float32)


def test_int8_exhaustive_vs_numpy(orc):
    c = np.arange(256, dtype=np.uint8)
    assert np.array_equal(orc.int8_to_f32(c), c.view(np.int8).astype(np.float32))


def test_int4_exhaustive_vs_shifts(orc):
    n = np.arange(16, dtype=np.uint8)
    got = orc.int4_to_f32(n)
    assert np.array_equal(got, _np_int4(n))
    assert got.min() == -8 and got.max() == 7 and got[15] == -1


def test_int4_nibble_order(orc):
    q = np.array([[0x71, 0x8F]], np.uint8)          # columns 0..3: 1, 7, -1, -8
    W = orc.dequant_int(orc.FMT_INT4_ROW, q, np.ones((1, 1), np.float32))
    assert W.tolist() == [[1.0, 7.0, -1.0, -8.0]]


def test_g64_group_index(orc):
    O, I = 3, 256
    q = np.full((O, I // 2), 0x11, np.uint8)        # every code 1
    s = np.array([[2.0 ** (o + 3 * g) for g in range(I // 64)] for o in range(O)], np.float32)
    W = orc.dequant_int(orc.FMT_INT4_G64, q, s)
    want = np.array([[2.0 ** (o + 3 * (i // 64)) for i in range(I)] for o in range(O)], np.float32)
    assert np.array_equal(W, want)


@pytest.mark.parametrize("fmt", [2, 3])
def test_per_row_scale_index(orc, fmt):
    O, I = 4, 96
    rng = np.random.default_rng(1)
    codes = rng.integers(-8, 8, size=(O, I))
    q = (codes & 0xFF).astype(np.uint8) if fmt == 2 else \
        ((codes[:, 0::2] & 15) | ((codes[:, 1::2] & 15) << 4)).astype(np.uint8)
    s = np.array([[2.0 ** -o] for o in range(O)], np.float32)
    W = orc.dequant_int(fmt, q, s)
    assert np.array_equal(W, (codes * 2.0 ** -np.arange(O)[:, None]).astype(np.float32))


def test_g64_with_equal_groups_is_per_row(orc):
    O, I = 5, 192
    rng = np.random.default_rng(2)
    q = rng.integers(0, 256, size=(O, I // 2), dtype=np.uint8)
    row = rng.uniform(0.5, 2.0, size=(O, 1)).astype(np.float32)
    a = orc.dequant_int(orc.FMT_INT4_ROW, q, row)
    b = orc.dequant_int(orc.FMT_INT4_G64, q, np.repeat(row, I // 64, axis=1))
    assert np.array_equal(a, b)


def test_int8_and_int4_agree_on_small_codes(orc):
    O, I = 3, 64
    codes = np.random.default_rng(3).integers(-8, 8, size=(O, I))
    q8 = (codes & 0xFF).astype(np.uint8)
    q4 = ((codes[:, 0::2] & 15) | ((codes[:, 1::2] & 15) << 4)).astype(np.uint8)
    s = np.random.default_rng(4).uniform(0.1, 1.0, size=(O, 1)).astype(np.float32)
    assert np.array_equal(orc.dequant_int(orc.FMT_INT8_ROW, q8, s), orc.dequant_int(orc.FMT_INT4_ROW, q4, s))


@pytest.mark.parametrize("fmt", [2, 3, 4])
def test_random_matrix_vs_numpy_decoder(orc, fmt):
    O, I = 6, 320
    rng = np.random.default_rng(5 + fmt)
    q = rng.integers(0, 256, size=(O, I if fmt == 2 else I // 2), dtype=np.uint8)
    s = rng.uniform(-2.0, 2.0, size=(O, I // 64 if fmt == 4 else 1)).astype(np.float32)
    assert np.array_equal(orc.dequant_int(fmt, q, s), _np_deq_int(fmt, q, s))


def test_rejects_bad_shapes(orc):
    with pytest.raises(ValueError):
        orc.dequant_int(orc.FMT_INT4_G64, np.zeros((2, 48), np.uint8), np.ones((2, 1), np.float32))  # I = 96
    with pytest.raises(ValueError):
        orc.dequant_int(7, np.zeros((2, 64), np.uint8), np.ones((2, 1), np.float32))


H, E, K, I = 256, 16, 2, 128


def _identity_expert(fmt, gate_scale):
    """Gate and up rows i select x_i (code 1), down row i selects h_i; the
    gate rows' scales are gate_scale, all others 1."""
    def enc(codes, scale):
        if fmt == syn.FMT_INT8_ROW:
            return (codes & 0xFF).astype(np.uint8), scale
        return ((codes[:, 0::2] & 15) | ((codes[:, 1::2] & 15) << 4)).astype(np.uint8), scale
    G = lambda cols: 64 if fmt == syn.FMT_INT4_G64 else cols
    gu = np.zeros((2 * I, H), np.int64)
    gu[np.arange(I), np.arange(I)] = 1
    gu[I + np.arange(I), np.arange(I)] = 1
    gs = np.ones((2 * I, H // G(H)), np.float32)
    gs[:I] = gate_scale
    dn = np.zeros((H, I), np.int64)
    dn[np.arange(I), np.arange(I)] = 1
    ds = np.ones((H, I // G(I)), np.float32)
    gq, gs = enc(gu, gs)
    dq, ds = enc(dn, ds)
    return gq, gs, dq, ds


@pytest.mark.parametrize("fmt", [2, 3, 4])
@pytest.mark.parametrize("gate_scale", [1.0, 0.5])
def test_identity_selection_expert(orc, fmt, gate_scale):
    L = orc.Layer(H, E, K, I, 0, fmt)
    g = torch.Generator().manual_seed(11)
    x = bits(torch.randn((H,), generator=g).to(torch.bfloat16))
    d = orc.expert_apply(L, orc.Expert(*_identity_expert(fmt, gate_scale)), I, x)
    xf = orc.bf16_to_f32(x).astype(np.float64)[:I]
    t = gate_scale * xf
    h = (t * scipy.special.expit(t) * xf).astype(np.float32).astype(np.float64)
    assert np.allclose(d[:I], h, rtol=1e-12, atol=0)
    assert np.all(d[I:] == 0)


def test_tiny_int4_g64_layer_vs_textbook(orc):
    wl = syn.WORKLOADS["tiny_i4g64"]
    W = syn.make_layer_weights(wl, 0)
    x = syn.make_x(wl, 0, 3)
    got = orc.layer_forward(oracle_layer(orc, wl, W), bits(x))
    ref = _textbook_layer(wl, W, bits(x), deq=lambda q, s: _np_deq_int(wl.fmt, host(q), host(s)))
    assert np.allclose(got["y"], ref, rtol=1e-5, atol=1e-6 * np.abs(ref).max())
