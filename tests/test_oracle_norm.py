"""Pins of the oracle's RMSNorm (the epilogue after the MoE output joins the
residual; GB10 blueprint, "Kernels": residual_add_rms_norm; Qwen3-8B card,
"Structure": RMSNorm over the hidden size) against closed forms and exact
symmetries, so that a dropped mean, a missing square root, eps in the wrong
place, a transposed weight or a sign error fails one of them."""
import numpy as np
import pytest

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def bf(orc, v):
    return orc.f32_to_bf16(np.asarray(v, np.float32))


def val(orc, bits):
    return orc.bf16_to_f32(bits)


def test_worked_example(orc):
    # x = (1, 2, 3, 4), gamma = 1, eps = 0: mean x^2 = 30/4 = 7.5, so
    # out_i = x_i / sqrt(7.5) = 0.36515, 0.73030, 1.09545, 1.46059; to bf16
    # (8 significant bits): 1.4609375 * 2^-2, 1.4609375 * 2^-1, 1.09375,
    # 1.4609375.
    x = bf(orc, [1, 2, 3, 4])[None, :]
    g = bf(orc, [1, 1, 1, 1])
    out = val(orc, orc.rms_norm(x, g, 0.0))[0]
    assert out.tolist() == [0.365234375, 0.73046875, 1.09375, 1.4609375]


@pytest.mark.parametrize("c", [0.5, -3.0, 17.25])
def test_constant_row(orc, c):
    # every x_o = c: mean x^2 = c^2, so out_o = gamma_o * c / |c| (eps = 0)
    H = 96
    rng = np.random.default_rng(1)
    gamma = bf(orc, rng.normal(size=H))
    out = orc.rms_norm(bf(orc, np.full(H, c))[None, :], gamma, 0.0)[0]
    assert np.array_equal(out, bf(orc, np.sign(c) * val(orc, gamma)))


def test_one_hot_row(orc):
    # x = a e_i: mean x^2 = a^2 / H, so out_i = gamma_i sqrt(H) sign(a), 0 elsewhere
    H, i, a = 64, 17, -2.5
    x = np.zeros(H, np.float32)
    x[i] = a
    gamma = bf(orc, np.linspace(0.5, 1.5, H))
    out = val(orc, orc.rms_norm(bf(orc, x)[None, :], gamma, 0.0)[0])
    want = np.zeros(H, np.float32)
    want[i] = val(orc, bf(orc, [val(orc, gamma[i]) * 8.0 * -1.0]))[0]     # sqrt(64) = 8
    assert np.array_equal(out, want)


def test_eps_inside_the_root(orc):
    # x = (3, 4) with eps = 12.5: mean x^2 = 12.5, so out = x / sqrt(25) = (0.6, 0.8)
    x = bf(orc, [3, 4])[None, :]
    out = val(orc, orc.rms_norm(x, bf(orc, [1, 1]), 12.5))[0]
    assert np.array_equal(out, val(orc, bf(orc, [0.6, 0.8])))


def test_exact_symmetries(orc):
    rng = np.random.default_rng(7)
    H = 257
    x = bf(orc, rng.normal(size=(3, H)))
    gamma = bf(orc, rng.normal(size=H))
    base = orc.rms_norm(x, gamma, 1e-6)
    # odd: negating x flips every sign bit
    neg = orc.rms_norm(x ^ np.uint16(0x8000), gamma, 1e-6)
    assert np.array_equal(neg, base ^ np.uint16(0x8000))
    # scale: 2x and x normalise to the same values when eps = 0 (exact in binary)
    a = orc.rms_norm(x, gamma, 0.0)
    b = orc.rms_norm(bf(orc, 2.0 * val(orc, x)), gamma, 0.0)
    assert np.array_equal(a, b)
    # weight: 2 gamma doubles the output exactly
    c = orc.rms_norm(x, bf(orc, 2.0 * val(orc, gamma)), 1e-6)
    assert np.array_equal(val(orc, c), 2.0 * val(orc, base))
    # permutation of the columns (with the weight) permutes the output
    p = rng.permutation(H)
    d = orc.rms_norm(x[:, p], gamma[p], 1e-6)
    assert np.array_equal(d, base[:, p])
    # rows are independent
    e = orc.rms_norm(x[1:2], gamma, 1e-6)
    assert np.array_equal(e[0], base[1])


def test_rejects_bad_arguments(orc):
    x = bf(orc, [1, 2])[None, :]
    with pytest.raises(ValueError):
        orc.rms_norm(x, bf(orc, [1, 1, 1]), 0.0)
    with pytest.raises(ValueError):
        orc.rms_norm(x, bf(orc, [1, 1]), -1.0)
