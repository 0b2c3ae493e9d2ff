"""Pins of the oracle's number-format decoders and block-scale indexing.

The decoders are checked exhaustively against torch's own casts (library
routines) and against the anchor values in tests/golden/formats.txt; the
block-scale layouts are pinned by one-hot probes that fail for a transposed
scale grid, a wrong block size or a swapped nibble order.
"""
import math
import os

import numpy as np
import pytest
import torch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "formats.txt")


def _golden():
    rows = []
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                fmt, code, val = line.split()
                rows.append((fmt, int(code, 16), float(val)))
    return rows


def _same(a, b):
    if math.isnan(b):
        return math.isnan(a)
    return a == b and math.copysign(1.0, a) == math.copysign(1.0, b)


@pytest.mark.parametrize("fmt,code,val", _golden())
def test_golden_anchor(orc, fmt, code, val):
    dec = {"e4m3": orc.e4m3_to_f32, "e2m1": orc.e2m1_to_f32, "bf16": orc.bf16_to_f32}[fmt]
    got = float(dec(np.array([code]))[0])
    assert _same(got, val), (fmt, hex(code), got, val)


def test_bf16_exhaustive_vs_torch(orc):
    bits = np.arange(1 << 16, dtype=np.uint16)
    ours = orc.bf16_to_f32(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float32).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_e4m3_exhaustive_vs_torch(orc):
    codes = np.arange(256, dtype=np.uint8)
    ours = orc.e4m3_to_f32(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    nan = np.isnan(ref)
    assert nan.sum() == 2  # 0x7f and 0xff only
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_e2m1_all_codes(orc):
    ours = orc.e2m1_to_f32(np.arange(16, dtype=np.uint8))
    mags = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    assert list(ours[:8]) == mags
    assert list(-ours[8:]) == mags


def test_bf16_rounding_vs_torch(orc):
    rng = np.random.default_rng(7)
    v = np.concatenate([rng.standard_normal(4000).astype(np.float32) * 10.0 ** rng.integers(-30, 30, 4000),
                        np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -(1.0 + 2.0 ** -8), 0.0, -0.0,
                                  3.4e38, 1e-45], np.float32)]).astype(np.float32)
    ours = orc.f32_to_bf16(v)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_fp8_dequant_matches_kron_formulation(orc):
    rng = np.random.default_rng(1)
    O, I = 256, 384
    q = rng.integers(0, 256, (O, I), dtype=np.uint8)
    q[(q & 0x7f) == 0x7f] = 0x11  # no NaN codes
    s = rng.uniform(0.5, 2.0, (O // 128, I // 128)).astype(np.float32)
    ref = torch.from_numpy(q).view(torch.float8_e4m3fn).to(torch.float64).numpy() * \
        np.kron(s.astype(np.float64), np.ones((128, 128)))
    W = orc.dequant_fp8(q, s)
    assert np.array_equal(W, ref.astype(np.float32))


@pytest.mark.parametrize("bi,bj", [(0, 0), (1, 2), (2, 1)])
def test_fp8_block_scale_one_hot(orc, bi, bj):
    O, I = 384, 384
    q = np.zeros((O, I), np.uint8)
    o, i = 128 * bi + 37, 128 * bj + 101
    q[o, i] = 0x40  # 2.0
    s = np.ones((O // 128, I // 128), np.float32)
    s[bi, bj] = 0.375
    W = orc.dequant_fp8(q, s)
    nz = np.argwhere(W != 0)
    assert nz.tolist() == [[o, i]]
    assert W[o, i] == np.float32(0.75)
    # a probe in a block whose scale is not the modified one keeps scale 1
    q2 = np.zeros_like(q)
    q2[128 * bj + 5, 128 * bi + 6] = 0x40
    W2 = orc.dequant_fp8(q2, s)
    expect = 0.75 if (bi == bj) else 2.0
    assert W2[128 * bj + 5, 128 * bi + 6] == np.float32(expect)


def test_nvfp4_layout_one_hot(orc):
    O, I = 4, 64
    q = np.zeros((O, I // 2), np.uint8)
    q[2, 5] = 0x3 | (0x5 << 4)     # column 10 -> code 3 (1.5), column 11 -> code 5 (3.0)
    sc = np.full((O, I // 16), 0x38, np.uint8)   # e4m3 1.0
    sc[2, 0] = 0x40                               # columns 0..15 of row 2 scaled by 2.0
    W = orc.dequant_nvfp4(q, sc, 0.25)
    nz = {tuple(p) for p in np.argwhere(W != 0)}
    assert nz == {(2, 10), (2, 11)}
    assert W[2, 10] == np.float32(1.5 * 2.0 * 0.25)
    assert W[2, 11] == np.float32(3.0 * 2.0 * 0.25)
    # same codes in the second group of 16 columns use that group's scale
    q2 = np.zeros_like(q)
    q2[2, 8] = 0x0a                               # column 16 -> -1.0, column 17 -> 0
    W2 = orc.dequant_nvfp4(q2, sc, 0.25)
    assert W2[2, 16] == np.float32(-0.25) and W2[2, 17] == 0


def test_nvfp4_dequant_matches_independent_formulation(orc):
    rng = np.random.default_rng(3)
    O, I = 32, 128
    q = rng.integers(0, 256, (O, I // 2), dtype=np.uint8)
    sc = rng.integers(0x20, 0x48, (O, I // 16), dtype=np.uint8)
    g = 0.0123
    mags = np.array([0, .5, 1, 1.5, 2, 3, 4, 6], np.float64)
    codes = np.empty((O, I), np.uint8)
    codes[:, 0::2] = q & 15
    codes[:, 1::2] = q >> 4
    val = mags[codes & 7] * np.where(codes & 8, -1.0, 1.0)
    scf = torch.from_numpy(sc).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ref = val * np.repeat(scf, 16, axis=1) * np.float64(np.float32(g))
    assert np.array_equal(orc.dequant_nvfp4(q, sc, g), ref.astype(np.float32))
