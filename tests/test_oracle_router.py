"""Pins for the router oracle (O5): a hand-worked case, the tie rule, the k = E
special case against scipy's softmax, invariants of the choice and the
weights, and the logit gradient against central finite differences and torch
autograd (an independent formulation of the same forward)."""
import math

import numpy as np
import pytest
import scipy.special
import torch

from oracle import router as R


def _logits(seed, T, E):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((T, E)).astype(np.float32)


def test_worked_example():
    # logits 2, 1, 0, -1 with k = 2: experts 0 and 1, weights e/(e+1), 1/(e+1)
    ids, w = R.route(np.array([[2.0, 1.0, 0.0, -1.0]], np.float32), 2)
    assert ids.tolist() == [[0, 1]]
    e = math.e
    assert np.allclose(w, [[e / (e + 1), 1 / (e + 1)]], rtol=0, atol=1e-15)


def test_tie_rule_and_slot_order():
    # equal logits: the lower index first; slots by descending logit
    ids, _ = R.route(np.array([[1.0, 3.0, 3.0, 0.0, 2.0]], np.float32), 3)
    assert ids.tolist() == [[1, 2, 4]]


def test_k_equal_e_is_softmax():
    l = _logits(1, 7, 9)
    ids, w = R.route(l, 9)
    ref = scipy.special.softmax(l.astype(np.float64), axis=1)
    got = np.zeros_like(ref)
    np.put_along_axis(got, ids.astype(np.int64), w, axis=1)
    assert np.allclose(got, ref, rtol=1e-14, atol=0)


@pytest.mark.parametrize("T,E,k", [(50, 8, 2), (20, 256, 8), (10, 512, 10), (5, 3, 1)])
def test_invariants(T, E, k):
    l = _logits(T * 1000 + E, T, E)
    ids, w = R.route(l, k)
    for t in range(T):
        chosen = set(ids[t].tolist())
        assert len(chosen) == k
        rest = [e for e in range(E) if e not in chosen]
        assert min(l[t, ids[t]]) >= (max(l[t, rest]) if rest else -np.inf)
        assert all(l[t, ids[t, j]] >= l[t, ids[t, j + 1]] for j in range(k - 1))
    assert np.all(w > 0) and np.all(w <= 1)
    assert np.allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-14)
    # shifting a row's logits changes nothing (the shift is exact in fp64)
    ids2, w2 = R.route(l.astype(np.float64) + 3.0, k)
    assert np.array_equal(ids, ids2) and np.allclose(w, w2, rtol=1e-12, atol=0)


def test_backward_finite_differences():
    T, E, k = 3, 6, 3
    l = _logits(7, T, E).astype(np.float64)
    c = np.random.default_rng(8).standard_normal((T, k))
    ids, _ = R.route(l, k)

    def loss(lv):
        _, w = R.route(lv, k)
        return float((w * c).sum())

    g = R.route_backward(l, ids, c)
    h = 1e-6
    fd = np.zeros_like(l)
    for t in range(T):
        for e in range(E):
            lp, lm = l.copy(), l.copy()
            lp[t, e] += h
            lm[t, e] -= h
            assert np.array_equal(R.route(lp, k)[0], ids) and np.array_equal(R.route(lm, k)[0], ids)
            fd[t, e] = (loss(lp) - loss(lm)) / (2 * h)
    assert np.abs(g - fd).max() <= 1e-6 * max(1.0, np.abs(fd).max())
    mask = np.zeros((T, E), bool)
    np.put_along_axis(mask, ids.astype(np.int64), True, axis=1)
    assert np.abs(g[~mask]).max() <= 1e-15              # unchosen experts get no gradient (up to rounding)
    assert np.allclose(g.sum(axis=1), 0, atol=1e-15)    # renormalised weights sum to 1


def test_backward_matches_autograd():
    T, E, k = 16, 32, 4
    l = _logits(9, T, E).astype(np.float64)
    dw = np.random.default_rng(10).standard_normal((T, k))
    ids, _ = R.route(l, k)
    lt = torch.tensor(l, dtype=torch.float64, requires_grad=True)
    p = torch.softmax(lt, dim=1)
    sel = torch.gather(p, 1, torch.tensor(ids, dtype=torch.int64))
    w = sel / sel.sum(dim=1, keepdim=True)
    (w * torch.tensor(dw)).sum().backward()
    assert np.allclose(R.route_backward(l, ids, dw), lt.grad.numpy(), rtol=1e-12, atol=1e-15)
