"""CPU checks of the tie inputs the GPU tie tests use (tests/helpers.py
tie_rows): each pattern holds the exact ties it promises, and the oracle's
top-k on them equals a brute-force ranking under the stated order (value
descending, the lower expert index first among equal values; +0 and -0 are
equal values)."""
import numpy as np
import pytest

from helpers import tie_rows


def test_patterns_hold_their_ties():
    E, k = 256, 8
    rows = tie_rows(E, k, 6, 11)
    assert np.all(rows[0] == rows[0][0])
    s1 = np.sort(rows[1])[::-1]
    assert s1[k - 2] == s1[k + 2] and s1[k - 3] != s1[k - 2]
    z = rows[2] == 0
    assert z.sum() == 2 * k and np.signbit(rows[2][z]).sum() == k
    top = rows[3] == rows[3].max()
    assert top.sum() == k + 2
    lanes = np.nonzero(top)[0]
    assert len({e % 64 // 16 for e in lanes}) == 4 and len({e // 64 for e in lanes}) >= 2
    s4 = np.sort(rows[4])[::-1]
    assert s4[0] == s4[2] != s4[3]
    assert len(np.unique(rows[5])) == E


@pytest.mark.parametrize("E,k", [(16, 2), (256, 8), (512, 10)])
def test_oracle_topk_on_tie_rows_is_the_stated_order(orc, E, k):
    rows = tie_rows(E, k, 12, 5 + E)
    ids, w = orc.topk_softmax(rows, k)
    for r in range(rows.shape[0]):
        # brute force: rank every expert by (-value, index); -0 == +0 as numbers
        key = sorted(range(E), key=lambda e: (-float(rows[r, e]), e))
        assert ids[r].tolist() == key[:k], r
        v = rows[r, key[:k]].astype(np.float64)
        p = np.exp(v - v.max())
        assert np.allclose(w[r], p / p.sum(), rtol=0, atol=1e-7)
