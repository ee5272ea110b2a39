"""Pins of the oracle's routing: top-k, gate weights, grouping."""
import numpy as np
import pytest
from scipy.special import softmax

from oracle import moe as M


def _brute_topk(row, k):
    chosen = []
    for _ in range(k):
        best = None
        for e, v in enumerate(row):
            if e in chosen:
                continue
            if best is None or v > row[best]:        # strict: earlier index wins ties
                best = e
        chosen.append(best)
    return chosen


@pytest.mark.parametrize("k", [1, 2, 3, 8])
def test_topk_brute_force_with_ties(k):
    rng = np.random.default_rng(k)
    z = rng.integers(-3, 4, size=(60, 8)).astype(np.float64)     # many exact ties
    ids = M.select_topk(z, k)
    for t in range(z.shape[0]):
        assert list(ids[t]) == _brute_topk(list(z[t]), k)


def test_topk_negative_zero_equals_zero():
    z = np.array([[-0.0, 0.0, -1.0]])
    assert list(M.select_topk(z, 2)[0]) == [0, 1]


def test_margin():
    z = np.array([[3.0, 1.0, 2.0, 2.5]])
    assert M.topk_margin(z, 2)[0] == pytest.approx(0.5)
    assert np.isinf(M.topk_margin(z, 4)[0])


def test_gate_weights_are_renormalised_full_softmax():
    rng = np.random.default_rng(2)
    z = rng.normal(0, 3, size=(40, 16))
    ids = M.select_topk(z, 4)
    w = M.gate_weights(z, ids)
    p = softmax(z, axis=1)                               # full softmax over E
    sel = np.take_along_axis(p, ids.astype(np.int64), axis=1)
    np.testing.assert_allclose(w, sel / sel.sum(axis=1, keepdims=True), rtol=1e-13, atol=0)
    np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-14)
    # k = E: weights are the plain softmax in descending order
    ids_all = M.select_topk(z, 16)
    np.testing.assert_allclose(M.gate_weights(z, ids_all), np.take_along_axis(p, ids_all.astype(np.int64), 1),
                               rtol=1e-13)


def test_router_logits_worked_example():
    # x = [1, 2] (exact bf16), R = [[1,0],[0,1],[1,1]], b = [0,0,0.5] -> z = [1, 2, 3.5]
    x = np.array([[0x3F80, 0x4000]], dtype=np.uint16)
    R = np.array([[1, 0], [0, 1], [1, 1]], dtype=np.float32)
    b = np.array([0, 0, 0.5], dtype=np.float32)
    assert list(M.router_logits(x, R, b)[0]) == [1.0, 2.0, 3.5]
    assert list(M.select_topk(M.router_logits(x, R, b), 2)[0]) == [2, 1]


def test_route_index_brute_force():
    rng = np.random.default_rng(3)
    T, E, k = 37, 10, 3
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    counts, offsets, perm_tok, perm_j, pos = M.route_index(ids, E)
    pairs = sorted((int(ids[t, j]), t, j) for t in range(T) for j in range(k))
    assert [p[1] for p in pairs] == list(perm_tok)
    assert [p[2] for p in pairs] == list(perm_j)
    assert list(counts) == list(np.bincount(ids.reshape(-1), minlength=E))
    assert offsets[0] == 0 and offsets[-1] == T * k
    for t in range(T):
        for j in range(k):
            assert perm_tok[pos[t, j]] == t and perm_j[pos[t, j]] == j
            e = ids[t, j]
            assert offsets[e] <= pos[t, j] < offsets[e + 1]
