"""Pins of the oracle's fp8 block-128 format with bf16 block scales (colibri
PR: a fixture of fp8 experts with BF16 128x128 block scales): the bf16 scale
widens exactly, so the matrix equals the f32-scale format holding the same
values; a one-hot scale block doubles exactly its 128x128 block; known bf16
patterns decode to their values; and a tiny layer agrees with a torch/numpy
float64 textbook layer.  A transposed scale index, a scale read as the low
half of a word or the wrong block size fails one of them."""
import numpy as np
import pytest
import torch

import moe_synth as syn
from helpers import bits, host, oracle_layer
from test_oracle_layer import _textbook_layer


def _bf(v):
    return torch.tensor(v, dtype=torch.float32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_equals_f32_scales_with_the_same_values(orc):
    rng = np.random.default_rng(1)
    O, I = 256, 384
    q = rng.integers(0, 256, size=(O, I), dtype=np.uint8)
    q[(q & 0x7F) == 0x7F] = 0
    sb = _bf(rng.uniform(0.01, 3.0, size=(2, 3)))
    sf = orc.bf16_to_f32(sb)
    assert np.array_equal(orc.dequant_fp8_bf16s(q, sb), orc.dequant_fp8(q, sf))


@pytest.mark.parametrize("bi,bj", [(0, 0), (1, 2), (0, 1)])
def test_one_hot_scale_block(orc, bi, bj):
    O, I = 256, 384
    q = np.full((O, I), 0x38, np.uint8)                 # e4m3 1.0
    s = np.full((2, 3), 0x3F80, np.uint16)              # bf16 1.0
    s[bi, bj] = 0x4000                                  # bf16 2.0
    W = orc.dequant_fp8_bf16s(q, s)
    want = np.ones((O, I), np.float32)
    want[bi * 128:(bi + 1) * 128, bj * 128:(bj + 1) * 128] = 2.0
    assert np.array_equal(W, want)


def test_known_bf16_scale_values(orc):
    q = np.full((128, 128), 0x38, np.uint8)
    for bits_, val in [(0x3F80, 1.0), (0x4040, 3.0), (0x3E00, 0.125), (0xBF00, -0.5), (0x3B80, 2.0 ** -8)]:
        W = orc.dequant_fp8_bf16s(q, np.array([[bits_]], np.uint16))
        assert np.all(W == val), hex(bits_)


def test_tiny_layer_vs_textbook(orc):
    wl = syn.WORKLOADS["tiny_f8bs"]
    W = syn.make_layer_weights(wl, 0)
    x = syn.make_x(wl, 0, 3)

    def deq(q, s):
        v = torch.from_numpy(host(q)).view(torch.float8_e4m3fn).to(torch.float64).numpy()
        sf = torch.from_numpy(host(s).view(np.int16)).view(torch.bfloat16).double().numpy()
        return (v * np.kron(sf, np.ones((128, 128)))).astype(np.float32)

    got = orc.layer_forward(oracle_layer(orc, wl, W), bits(x))
    ref = _textbook_layer(wl, W, bits(x), deq=deq)
    assert np.allclose(got["y"], ref, rtol=1e-5, atol=1e-6 * np.abs(ref).max())
