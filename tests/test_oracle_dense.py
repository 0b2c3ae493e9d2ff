"""Pins of the oracle's dense fp8 block-128 projection (GB10 blueprint,
"Kernels": w8a16_gemm_pipelined_m32; "Precision": fp8/block128x128 weights
read bf16 activations): y = x . dequant(W)^T, against closed forms: the
identity, a permutation, power-of-two block scales (one per 128x128 block,
row block n/128 by column block k/128), a one-hot row, and exact scaling.  A
transposed product, a swapped scale index or a wrong block size fails one."""
import numpy as np
import pytest

E4M3_ONE = 0x38      # e4m3: sign 0, exponent 7 (bias 7), mantissa 0 -> 1.0


def bf(orc, v):
    return orc.f32_to_bf16(np.asarray(v, np.float32))


def xval(orc, bits):
    return orc.bf16_to_f32(bits).astype(np.float64)


def test_identity(orc):
    n = 128
    q = np.zeros((n, n), np.uint8)
    np.fill_diagonal(q, E4M3_ONE)
    s = np.ones((1, 1), np.float32)
    x = bf(orc, np.random.default_rng(0).normal(size=(3, n)))
    assert np.array_equal(orc.dense_fp8(q, s, x), xval(orc, x))


def test_permutation(orc):
    n = 256
    p = np.random.default_rng(1).permutation(n)
    q = np.zeros((n, n), np.uint8)
    q[np.arange(n), p] = E4M3_ONE           # row j picks column p[j]
    s = np.ones((2, 2), np.float32)
    x = bf(orc, np.random.default_rng(2).normal(size=(2, n)))
    assert np.array_equal(orc.dense_fp8(q, s, x), xval(orc, x)[:, p])


def test_block_scales(orc):
    # every code 1.0; scale of block (nb, kb) = 2^(nb - 2 kb): y[n] is the sum
    # over column blocks of that scale times the block's sum of x
    N, K = 256, 384
    q = np.full((N, K), E4M3_ONE, np.uint8)
    s = np.array([[2.0 ** (nb - 2 * kb) for kb in range(3)] for nb in range(2)], np.float32)
    x = bf(orc, np.random.default_rng(3).normal(size=(2, K)))
    xv = xval(orc, x)
    block_sums = xv.reshape(2, 3, 128).sum(axis=2)                  # [R][kb]
    want = np.stack([block_sums @ s[n // 128].astype(np.float64) for n in range(N)], axis=1)
    assert np.allclose(orc.dense_fp8(q, s, x), want, rtol=1e-12, atol=1e-12)


def test_one_hot_row_selects_a_column(orc):
    N, K, k = 128, 256, 200
    rng = np.random.default_rng(4)
    q = rng.integers(0, 256, size=(N, K), dtype=np.uint8)
    q[(q & 0x7F) == 0x7F] = 0                                       # no NaN codes
    s = np.array([[0.5, 4.0]], np.float32)
    x = np.zeros((1, K), np.uint16)
    x[0, k] = bf(orc, [1.0])[0]
    y = orc.dense_fp8(q, s, x)[0]
    # column k of the dequantised matrix: code value times its block's scale
    col = orc.e4m3_to_f32(q[:, k]).astype(np.float64) * 4.0           # k = 200 is in column block 1
    assert np.array_equal(y, col)


def test_exact_scaling(orc):
    rng = np.random.default_rng(5)
    N, K = 256, 256
    q = rng.integers(0, 256, size=(N, K), dtype=np.uint8)
    q[(q & 0x7F) == 0x7F] = 0
    s = rng.uniform(0.5, 2.0, size=(2, 2)).astype(np.float32)
    x = bf(orc, rng.normal(size=(3, K)))
    y = orc.dense_fp8(q, s, x)
    x2 = bf(orc, 2.0 * xval(orc, x))
    assert np.array_equal(orc.dense_fp8(q, s, x2), 2.0 * y)
    s2 = (2.0 * s).astype(np.float32)
    assert np.array_equal(orc.dense_fp8(q, s2, x), 2.0 * y)


def test_rejects_bad_shapes(orc):
    q = np.zeros((128, 100), np.uint8)
    with pytest.raises(ValueError):
        orc.dense_fp8(q, np.ones((1, 1), np.float32), np.zeros((1, 100), np.uint16))
