"""Seeded generators: reproducible, shaped like the pages' models, encoders
within half a quantisation step, routing statistics as intended."""
import os

import numpy as np
import torch

import moe_synth as syn
from helpers import min_top_gap, router_only_layer, tie_free_x, bits

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_shapes.txt")


def test_shapes_match_the_pages():
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, val = line.split()
            name, field = key.split(".")
            assert getattr(syn.WORKLOADS[name], field) == int(val), key


def test_reproducible_and_distinct():
    wl = syn.WORKLOADS["tiny"]
    a = syn.make_layer_weights(wl, 0)
    b = syn.make_layer_weights(wl, 0)
    c = syn.make_layer_weights(wl, 1)
    for k in a:
        if a[k] is not None:
            assert torch.equal(a[k], b[k]), k
    assert not torch.equal(a["gu_q"], c["gu_q"])
    assert torch.equal(syn.make_x(wl, 0, 2, 0), syn.make_x(wl, 0, 2, 0))
    assert not torch.equal(syn.make_x(wl, 0, 2, 0), syn.make_x(wl, 0, 2, 1))


def test_fp8_encoder_error_within_half_step():
    w = torch.randn(3, 256, 384) * 0.02
    q, s = syn.quant_fp8_b128(w)
    dec = q.view(torch.float8_e4m3fn).float() * s.repeat_interleave(128, 1).repeat_interleave(128, 2)
    # e4m3 has 3 mantissa bits: relative spacing 2^-3, half-step 2^-4; subnormal step 2^-9*scale
    tol = torch.maximum(w.abs() * 2.0 ** -4, s.repeat_interleave(128, 1).repeat_interleave(128, 2) * 2.0 ** -10)
    assert torch.all((dec - w).abs() <= tol * 1.0001)
    assert int((q & 0x7f).max()) <= 0x7e


def test_nvfp4_encoder_error_bound():
    w = torch.randn(2, 64, 256) * 0.02
    q, sc, g = syn.quant_nvfp4(w)
    mags = torch.tensor([0, .5, 1, 1.5, 2, 3, 4, 6])
    codes = torch.stack([q & 15, q >> 4], -1).reshape(2, 64, 256).long()
    val = mags[codes & 7] * torch.where(codes >= 8, -1.0, 1.0)
    scale = sc.view(torch.float8_e4m3fn).float().repeat_interleave(16, -1) * g[:, None, None]
    dec = val * scale
    # nearest e2m1 magnitude: error at most half the widest gap (2 between 4 and 6) in code units
    assert torch.all((dec - w).abs() <= scale * 1.0 + 1e-12)
    rel = (dec - w).norm() / w.norm()
    assert rel < 0.12


def test_rms_normalised_activations():
    wl = syn.WORKLOADS["a3b"]
    x = syn.make_x(wl, 3, 4).float()
    rms = x.pow(2).mean(-1).sqrt()
    assert torch.allclose(rms, torch.ones(4), atol=1e-2)


def test_uniform_and_zipf_logits():
    u = syn.make_logits_in(syn.WORKLOADS["a3b_multi"], 0, 64)
    assert u.shape == (64, 256) and float(u.min()) >= 0 and float(u.max()) < 1
    z = syn.make_logits_in(syn.WORKLOADS["a3b_zipf"], 0, 512)
    counts = torch.bincount(z.topk(8, dim=1).indices.flatten(), minlength=256)
    assert counts.sum() == 512 * 8
    assert counts.max() >= 256          # hot experts take most rows
    assert (counts <= 1).sum() >= 20    # and a long tail is nearly idle


def test_tie_free_redraw(orc):
    wl = syn.WORKLOADS["a3b"]
    g = torch.Generator().manual_seed(5)
    W = {"router_bias": None,
         "router_w": (torch.randn((wl.n_experts, wl.hidden), generator=g) * 0.02).to(torch.bfloat16)}
    x, attempt = tie_free_x(orc, wl, W, 0, 1)
    logits = orc.router_logits(router_only_layer(orc, wl, W), bits(x))
    assert min_top_gap(logits, wl.top_k) >= 1e-3


def test_effective_bytes_of_the_35b_row():
    wl = syn.WORKLOADS["a3b"]
    assert syn.effective_weight_bytes(wl, 8, True) == 29_371_136
    # 397B-A17B NVFP4 expert: 7,077,896 bytes including two f32 globals
    wl4 = syn.WORKLOADS["a17b"]
    one = syn.effective_weight_bytes(wl4, 1, False) - syn.effective_weight_bytes(wl4, 0, False)
    assert one == 7_077_896
    assert np.isclose(syn.expected_distinct(syn.WORKLOADS["a3b_multi"], 64), 222.44, atol=0.01)
