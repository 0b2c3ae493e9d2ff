"""Pins of the oracle's expert FFN, shared gate, blend and whole layer.

Closed forms: the zero expert; an identity-selection expert whose output is
silu(x_i) * x_i on the first I coordinates; a zero shared-gate vector (s = 1/2
exactly); identical routed experts (the blend no longer depends on routing);
all-zero weights leave the residual bit-unchanged; relabelling experts maps ids
and leaves y bit-identical.  A textbook SwiGLU written with numpy float64 and
torch's format casts checks a random tiny layer end to end.
"""
import numpy as np
import pytest
import scipy.special
import torch

import moe_synth as syn
from helpers import bits, host, oracle_layer

H, E, K, I = 256, 16, 2, 128


def _fp8_identity_expert(orc, inter, hidden, gate_scale=1.0):
    gu = np.zeros((2 * inter, hidden), np.uint8)
    gu[np.arange(inter), np.arange(inter)] = 0x38            # e4m3 1.0
    gu[inter + np.arange(inter), np.arange(inter)] = 0x38
    gu_s = np.ones((2 * inter // 128, hidden // 128), np.float32)
    gu_s[: inter // 128, :] = gate_scale
    dn = np.zeros((hidden, inter), np.uint8)
    dn[np.arange(inter), np.arange(inter)] = 0x38
    dn_s = np.ones((hidden // 128, inter // 128), np.float32)
    return orc.Expert(gu, gu_s, dn, dn_s)


def _nvfp4_identity_expert(orc, inter, hidden, g):
    codes = np.zeros((2 * inter, hidden), np.uint8)
    codes[np.arange(inter), np.arange(inter)] = 0x2          # e2m1 1.0
    codes[inter + np.arange(inter), np.arange(inter)] = 0x2
    gu = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    dcodes = np.zeros((hidden, inter), np.uint8)
    dcodes[np.arange(inter), np.arange(inter)] = 0x2
    dn = (dcodes[:, 0::2] | (dcodes[:, 1::2] << 4)).astype(np.uint8)
    gu_s = np.full((2 * inter, hidden // 16), 0x40, np.uint8)  # e4m3 2.0
    dn_s = np.full((hidden, inter // 16), 0x40, np.uint8)
    return orc.Expert(gu, gu_s, dn, dn_s, gu_g=g, dn_g=g)


def _x(seed, rows=1, hidden=H):
    g = torch.Generator().manual_seed(seed)
    return bits(torch.randn((rows, hidden), generator=g).to(torch.bfloat16))


def _silu(t):
    return t * scipy.special.expit(t)


def test_zero_expert_gives_zero(orc):
    L = orc.Layer(H, E, K, I, 0, 0)
    X = orc.Expert(np.zeros((2 * I, H), np.uint8), np.ones((2 * I // 128, H // 128), np.float32),
                   np.zeros((H, I), np.uint8), np.ones((H // 128, I // 128), np.float32))
    d = orc.expert_apply(L, X, I, _x(1)[0])
    assert np.all(d == 0)


@pytest.mark.parametrize("gate_scale", [1.0, 0.5, 2.0])
def test_identity_selection_expert(orc, gate_scale):
    L = orc.Layer(H, E, K, I, 0, 0)
    x = _x(2)[0]
    d = orc.expert_apply(L, _fp8_identity_expert(orc, I, H, gate_scale), I, x)
    xf = orc.bf16_to_f32(x).astype(np.float64)[:I]
    h = (_silu(gate_scale * xf) * xf).astype(np.float32).astype(np.float64)
    assert np.allclose(d[:I], h, rtol=1e-12, atol=0)
    assert np.all(d[I:] == 0)


def test_identity_selection_expert_nvfp4(orc):
    L = orc.Layer(H, E, K, I, 0, 1)
    x = _x(3)[0]
    d = orc.expert_apply(L, _nvfp4_identity_expert(orc, I, H, 0.5), I, x)   # 1.0 * 2.0 * 0.5
    xf = orc.bf16_to_f32(x).astype(np.float64)[:I]
    h = (_silu(xf) * xf).astype(np.float32).astype(np.float64)
    assert np.allclose(d[:I], h, rtol=1e-12, atol=0)
    assert np.all(d[I:] == 0)


def _tiny():
    wl = syn.WORKLOADS["tiny"]
    return wl, syn.make_layer_weights(wl, 0)


def _textbook_layer(wl, W, x_bits, logits=None, residual=None, deq=None):
    """Independent float64 formulation: numpy matmuls over weights decoded by
    torch's e4m3 cast (or the given decoder), scipy softmax, python sort."""
    if deq is None:
        def deq(q, s):
            v = torch.from_numpy(host(q)).view(torch.float8_e4m3fn).to(torch.float64).numpy()
            return (v * np.kron(host(s).astype(np.float64), np.ones((128, 128)))).astype(np.float32)

    xf = torch.from_numpy(x_bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    if logits is None:
        wr = W["router_w"].double().numpy()
        logits = (xf @ wr.T).astype(np.float32) + host(W["router_bias"])
    p = scipy.special.softmax(logits.astype(np.float64), axis=1)
    R = xf.shape[0]
    y = np.zeros((R, wl.hidden))
    for r in range(R):
        order = sorted(range(wl.n_experts), key=lambda e: (-p[r, e], e))[: wl.top_k]
        wsel = p[r, order] / p[r, order].sum()

        def ffn(gq, gs, dq, ds, inter):
            a = deq(gq, gs).astype(np.float64) @ xf[r]
            h = (_silu(a[:inter]) * a[inter:]).astype(np.float32).astype(np.float64)
            return deq(dq, ds).astype(np.float64) @ h

        for j, e in enumerate(order):
            y[r] += float(np.float32(wsel[j])) * ffn(W["gu_q"][e], W["gu_s"][e], W["dn_q"][e],
                                                      W["dn_s"][e], wl.inter)
        s = scipy.special.expit(xf[r] @ W["shared_gate_w"].double().numpy())
        y[r] += float(np.float32(s)) * ffn(W["sh_gu_q"][0], W["sh_gu_s"][0], W["sh_dn_q"][0],
                                           W["sh_dn_s"][0], wl.shared_inter)
    return y


def test_tiny_layer_vs_textbook(orc):
    wl, W = _tiny()
    x = syn.make_x(wl, 0, 4)
    L = oracle_layer(orc, wl, W)
    got = orc.layer_forward(L, bits(x))
    ref = _textbook_layer(wl, W, bits(x))
    assert np.allclose(got["y"], ref, rtol=1e-5, atol=1e-6 * np.abs(ref).max())


def test_tiny_layer_with_logits_in_vs_textbook(orc):
    wl, W = _tiny()
    x = syn.make_x(wl, 0, 3)
    logits = np.random.default_rng(4).uniform(0, 1, (3, wl.n_experts)).astype(np.float32)
    got = orc.layer_forward(oracle_layer(orc, wl, W), bits(x), logits_in=logits)
    ref = _textbook_layer(wl, W, bits(x), logits=logits)
    assert np.allclose(got["y"], ref, rtol=1e-5, atol=1e-6 * np.abs(ref).max())


def test_zero_shared_gate_vector_gives_one_half(orc):
    wl, W = _tiny()
    W = dict(W)
    W["shared_gate_w"] = torch.zeros_like(W["shared_gate_w"])
    out = orc.layer_forward(oracle_layer(orc, wl, W), bits(syn.make_x(wl, 0, 2)))
    assert np.all(out["s"] == np.float32(0.5))


def test_zero_shared_expert_leaves_routed_part(orc):
    wl, W = _tiny()
    x = bits(syn.make_x(wl, 0, 2))
    Wz = dict(W)
    Wz["sh_gu_q"] = torch.zeros_like(W["sh_gu_q"])
    with_zero = orc.layer_forward(oracle_layer(orc, wl, Wz), x)
    L0 = oracle_layer(orc, wl, W)
    no_shared = orc.Layer(wl.hidden, wl.n_experts, wl.top_k, wl.inter, 0, wl.fmt,
                          router_w=L0.router_w, router_bias=L0.router_bias,
                          experts={e: orc.Expert(host(W["gu_q"][e]), host(W["gu_s"][e]),
                                                 host(W["dn_q"][e]), host(W["dn_s"][e]))
                                   for e in range(wl.n_experts)})
    ref = orc.layer_forward(no_shared, x)
    assert np.array_equal(with_zero["y"], ref["y"])
    assert np.array_equal(with_zero["ids"], ref["ids"])


def test_identical_experts_make_routing_irrelevant(orc):
    wl, W = _tiny()
    W = dict(W)
    for key in ("gu_q", "gu_s", "dn_q", "dn_s"):
        W[key] = W[key][:1].expand_as(W[key]).contiguous()
    x = bits(syn.make_x(wl, 0, 3))
    L = oracle_layer(orc, wl, W)
    rng = np.random.default_rng(21)
    a = orc.layer_forward(L, x, logits_in=rng.standard_normal((3, E)).astype(np.float32))
    b = orc.layer_forward(L, x, logits_in=rng.standard_normal((3, E)).astype(np.float32))
    assert not np.array_equal(a["ids"], b["ids"])
    assert np.allclose(a["y"], b["y"], rtol=1e-6, atol=1e-7)
    X0 = orc.Expert(host(W["gu_q"][0]), host(W["gu_s"][0]), host(W["dn_q"][0]), host(W["dn_s"][0]))
    Xs = orc.Expert(host(W["sh_gu_q"][0]), host(W["sh_gu_s"][0]), host(W["sh_dn_q"][0]),
                    host(W["sh_dn_s"][0]))
    for r in range(3):
        ref = orc.expert_apply(L, X0, I, x[r]) + float(a["s"][r]) * orc.expert_apply(L, Xs, I, x[r])
        assert np.allclose(a["y"][r], ref, rtol=1e-6, atol=1e-7)


def test_all_zero_weights_leave_residual_unchanged(orc):
    wl, W = _tiny()
    Wz = {k: (torch.zeros_like(v) if (v is not None and k.endswith("_q")) else v)
          for k, v in W.items()}
    x = bits(syn.make_x(wl, 0, 3))
    res = bits(syn.make_residual(wl, 0, 3))
    out = orc.layer_forward(oracle_layer(orc, wl, Wz), x, residual=res)
    assert np.all(out["y"] == 0)
    assert np.array_equal(out["out"], res)


def test_residual_blend_single_rounding(orc):
    wl, W = _tiny()
    x = bits(syn.make_x(wl, 0, 2))
    res = bits(syn.make_residual(wl, 0, 2))
    a = orc.layer_forward(oracle_layer(orc, wl, W), x, residual=res)
    b = orc.layer_forward(oracle_layer(orc, wl, W), x)
    ref = (torch.from_numpy(a["y"]).double() +
           torch.from_numpy(res.view(np.int16)).view(torch.bfloat16).double())
    ref_bits = bits(ref.float().to(torch.bfloat16))
    assert np.array_equal(a["out"], ref_bits)
    assert np.array_equal(b["out"], bits(torch.from_numpy(b["y"]).to(torch.bfloat16)))


def test_expert_relabelling_invariance(orc):
    wl, W = _tiny()
    x = bits(syn.make_x(wl, 0, 3))
    base = orc.layer_forward(oracle_layer(orc, wl, W), x)
    pi = np.random.default_rng(31).permutation(E)       # expert e becomes pi[e]
    inv = np.argsort(pi)
    Wp = dict(W)
    for key in ("router_w", "router_bias", "gu_q", "gu_s", "dn_q", "dn_s"):
        Wp[key] = W[key][torch.from_numpy(inv)]
    permuted = orc.layer_forward(oracle_layer(orc, wl, Wp), x)
    # the bias follows its expert, so logits are relabelled exactly
    assert np.array_equal(pi[base["ids"]], permuted["ids"])
    assert np.array_equal(base["w"], permuted["w"])
    assert np.array_equal(base["y"], permuted["y"])


def test_rejects_missing_expert(orc):
    wl, W = _tiny()
    x = bits(syn.make_x(wl, 0, 1))
    L = oracle_layer(orc, wl, W, experts=[0])
    with pytest.raises(ValueError):
        orc.layer_forward(L, x)
