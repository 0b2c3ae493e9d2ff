"""Pins of the oracle's router GEMV, top-k softmax and grouping.

Top-k is checked by brute force over every k-subset on small expert counts,
softmax/renormalisation by closed forms (E == k, k == 1, shift invariance,
softmax over the chosen logits), grouping against numpy's stable argsort.
"""
import itertools

import numpy as np
import pytest
import scipy.special

import moe_synth as syn
from helpers import bits, router_only_layer


def test_router_logits_vs_float64_matmul(orc):
    wl = syn.WORKLOADS["tiny"]
    W = syn.make_layer_weights(wl, 0)
    x = syn.make_x(wl, 0, 3)
    got = orc.router_logits(router_only_layer(orc, wl, W), bits(x))
    xf = x.float().double().numpy()
    wr = W["router_w"].float().double().numpy()
    terms = np.abs(xf) @ np.abs(wr).T
    ref = xf @ wr.T
    ref32 = ref.astype(np.float32) + W["router_bias"].numpy()
    assert np.all(np.abs(got - ref32) <= 1e-6 * terms + 1e-7)
    # the bias is present and is 1e-3 * e
    got_nb = orc.router_logits(orc.Layer(wl.hidden, wl.n_experts, wl.top_k, wl.inter, 0, 0,
                                         router_w=bits(W["router_w"])), bits(x))
    assert np.allclose(got - got_nb, 1e-3 * np.arange(wl.n_experts)[None, :], atol=1e-6)


@pytest.mark.parametrize("E,k", [(4, 1), (6, 2), (8, 3), (10, 4), (12, 5), (12, 12), (7, 7)])
def test_topk_brute_force(orc, E, k):
    rng = np.random.default_rng(E * 100 + k)
    logits = rng.standard_normal((20, E)).astype(np.float32)
    ids, w = orc.topk_softmax(logits, k)
    for r in range(logits.shape[0]):
        best = max(itertools.combinations(range(E), k),
                   key=lambda S: sum(float(logits[r, e]) for e in S))
        assert set(ids[r].tolist()) == set(best)
        # descending order of value
        assert np.all(np.diff(logits[r, ids[r]]) <= 0)


def test_topk_forced_ties_lower_index_wins(orc):
    E, k = 10, 4
    logits = np.array([[0, 1, 1, 1, 0.5, 1, 0.5, 0, 2, 1],
                       [3, 3, 3, 3, 3, 3, 3, 3, 3, 3],
                       [0, 0, 0, 0, 0, 0, 0, 5, 5, 0]], np.float32)
    ids, w = orc.topk_softmax(logits, k)
    for r in range(logits.shape[0]):
        chosen = set(ids[r].tolist())
        for e in chosen:
            for f in set(range(E)) - chosen:
                assert logits[r, e] > logits[r, f] or (logits[r, e] == logits[r, f] and e < f)
        for a, b in zip(ids[r][:-1], ids[r][1:]):
            assert logits[r, a] > logits[r, b] or (logits[r, a] == logits[r, b] and a < b)
    assert ids[1].tolist() == [0, 1, 2, 3]
    assert np.all(w[1] == np.float32(0.25))


def test_renormalised_weights_are_softmax_of_chosen_logits(orc):
    rng = np.random.default_rng(5)
    for E, k in [(16, 2), (256, 8), (512, 10)]:
        logits = (rng.standard_normal((8, E)) * 2).astype(np.float32)
        ids, w = orc.topk_softmax(logits, k)
        assert np.allclose(w.sum(axis=1), 1.0, atol=1e-6)
        chosen = np.take_along_axis(logits, ids, axis=1).astype(np.float64)
        ref = scipy.special.softmax(chosen, axis=1)
        assert np.allclose(w, ref, rtol=1e-6, atol=1e-7)


def test_full_softmax_when_k_equals_E(orc):
    rng = np.random.default_rng(9)
    logits = rng.standard_normal((5, 9)).astype(np.float32)
    ids, w = orc.topk_softmax(logits, 9)
    ref = scipy.special.softmax(logits.astype(np.float64), axis=1)
    assert np.allclose(w, np.take_along_axis(ref, ids, axis=1), rtol=1e-6)


def test_k1_weight_is_exactly_one(orc):
    rng = np.random.default_rng(11)
    logits = rng.standard_normal((7, 32)).astype(np.float32)
    ids, w = orc.topk_softmax(logits, 1)
    assert np.all(w == 1.0)
    assert np.array_equal(ids[:, 0], np.argmax(logits, axis=1))


def test_shift_invariance(orc):
    rng = np.random.default_rng(12)
    logits = rng.standard_normal((6, 64)).astype(np.float32)
    ids0, w0 = orc.topk_softmax(logits, 8)
    ids1, w1 = orc.topk_softmax(logits + np.float32(3.0), 8)
    assert np.array_equal(ids0, ids1)
    assert np.allclose(w0, w1, atol=2e-6)


def test_expert_relabelling_maps_ids(orc):
    rng = np.random.default_rng(13)
    E, k = 40, 6
    logits = rng.standard_normal((9, E)).astype(np.float32)
    pi = rng.permutation(E)              # expert e is renamed pi[e]
    relabelled = np.empty_like(logits)
    relabelled[:, pi] = logits
    ids0, w0 = orc.topk_softmax(logits, k)
    ids1, w1 = orc.topk_softmax(relabelled, k)
    assert np.array_equal(pi[ids0], ids1)
    assert np.array_equal(w0, w1)


@pytest.mark.parametrize("R,E,k", [(1, 16, 2), (5, 16, 2), (64, 256, 8), (512, 256, 8),
                                   (8, 512, 10), (3, 4, 4)])
def test_grouping_vs_stable_argsort(orc, R, E, k):
    rng = np.random.default_rng(R * 7 + E)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(R)]).astype(np.int32)
    counts, offsets, perm = orc.group(ids, E)
    flat = ids.ravel()
    assert np.array_equal(counts, np.bincount(flat, minlength=E))
    assert offsets[0] == 0 and offsets[-1] == R * k
    assert np.array_equal(np.diff(offsets), counts)
    assert np.array_equal(perm, np.argsort(flat, kind="stable"))
    assert np.array_equal(np.sort(perm), np.arange(R * k))
    for e in range(E):
        seg = perm[offsets[e]:offsets[e + 1]]
        assert np.all(flat[seg] == e)
        assert np.all(np.diff(seg // k) > 0)


def test_grouping_empty_rows(orc):
    counts, offsets, perm = orc.group(np.zeros((0, 4), np.int32), 16)
    assert counts.sum() == 0 and np.all(offsets == 0) and perm.size == 0
