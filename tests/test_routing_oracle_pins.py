"""Pins of the router / routing-statistics oracle to things other than itself:
a hand-worked example, scalar brute force, a library softmax, invariants of a
top-k softmax router, and planted mistakes that the pins must catch."""
import math

import numpy as np
import pytest
from scipy.special import softmax as scipy_softmax

import oracle.routing_oracle as ro


def f16(a):
    return np.asarray(a, dtype=np.float16)


# --- brute force written for the tests only --------------------------------
def route_bruteforce(x, wr, k):
    T, H = x.shape
    E = wr.shape[0]
    ids, ws = [], []
    for t in range(T):
        logit = [math.fsum(float(x[t, h]) * float(wr[e, h]) for h in range(H)) for e in range(E)]
        left = list(range(E))
        chosen = []
        for _ in range(k):
            best = left[0]
            for e in left[1:]:
                if logit[e] > logit[best]:   # strict: an equal logit keeps the lower id
                    best = e
            chosen.append(best)
            left.remove(best)
        m = logit[chosen[0]]
        z = [math.exp(logit[e] - m) for e in chosen]
        s = math.fsum(z)
        ids.append(chosen)
        ws.append([v / s for v in z])
    return np.array(ids), np.array(ws)


def test_hand_worked_example():
    # Wr rows: e0 = [0, 1], e1 = [1, 0], e2 = [2, 0], e3 = [-1, 0]; k = 2.
    #  x = [1, 0]: logits [0, 1, 2, -1] -> ids [2, 1], w = [e/(e+1), 1/(e+1)]
    #  x = [0, 0]: all logits 0 (ties)  -> ids [0, 1], w = [1/2, 1/2]
    #  x = [1, 1]: logits [1, 1, 2, -1] -> ids [2, 0] (e0, e1 tie: lower id), w as the first token
    wr = f16([[0, 1], [1, 0], [2, 0], [-1, 0]])
    x = f16([[1, 0], [0, 0], [1, 1]])
    ids, w, _ = ro.route(x, wr, 2)
    e = math.e
    assert ids.tolist() == [[2, 1], [0, 1], [2, 0]]
    np.testing.assert_allclose(w, [[e / (e + 1), 1 / (e + 1)], [0.5, 0.5], [e / (e + 1), 1 / (e + 1)]],
                               rtol=0, atol=1e-15)
    count, mass = ro.routing_stats(ids, w, 4)
    assert count.tolist() == [2, 2, 2, 0]
    a, b = e / (e + 1), 1 / (e + 1)
    # e0: token 1 (1/2) + token 2 slot 1 (b); e1: token 0 slot 1 (b) + token 1 (1/2); e2: a twice
    np.testing.assert_allclose(mass, [0.5 + b, b + 0.5, 2 * a, 0.0], rtol=0, atol=1e-15)


@pytest.mark.parametrize("T,H,E,k,seed", [(5, 16, 7, 3, 0), (4, 32, 3, 3, 1), (6, 8, 9, 1, 2)])
def test_bruteforce(T, H, E, k, seed):
    rng = np.random.default_rng(seed)
    x = f16(rng.standard_normal((T, H)))
    wr = f16(rng.normal(0, 0.5, (E, H)))
    ids, w, _ = ro.route(x, wr, k)
    bi, bw = route_bruteforce(x, wr, k)
    assert np.array_equal(ids, bi)
    np.testing.assert_allclose(w, bw, rtol=0, atol=1e-12)


def test_invariants_and_library_softmax():
    rng = np.random.default_rng(3)
    T, H, E, k = 40, 64, 12, 4
    x = f16(rng.standard_normal((T, H)))
    wr = f16(rng.normal(0, 0.2, (E, H)))
    ids, w, logits = ro.route(x, wr, k)
    np.testing.assert_allclose(w.sum(axis=1), 1.0, atol=1e-14)
    assert np.all(np.diff(w, axis=1) <= 1e-15)                       # descending weights
    for t in range(T):
        assert len(set(ids[t].tolist())) == k
        rest = np.setdiff1d(np.arange(E), ids[t])
        assert logits[t, ids[t]].min() >= logits[t, rest].max()
    # softmax over the selected logits = the library softmax of that slice
    sel = np.take_along_axis(logits, ids.astype(np.int64), axis=1)
    np.testing.assert_allclose(w, scipy_softmax(sel, axis=1), rtol=1e-13)
    # k = E: every expert, softmax over all logits, order = stable argsort
    ids_all, w_all, _ = ro.route(x, wr, E)
    assert np.array_equal(ids_all, np.argsort(-logits, axis=1, kind="stable"))
    np.testing.assert_allclose(np.take_along_axis(w_all, np.argsort(ids_all, axis=1), axis=1),
                               scipy_softmax(logits, axis=1), rtol=1e-13)
    # statistics: library histogram, totals
    count, mass = ro.routing_stats(ids, w, E)
    assert np.array_equal(count, np.bincount(ids.reshape(-1), minlength=E))
    np.testing.assert_allclose(mass, np.bincount(ids.reshape(-1), weights=w.reshape(-1), minlength=E), atol=1e-13)
    assert count.sum() == T * k
    assert abs(mass.sum() - T) < 1e-12


def test_x_zero_gives_lowest_ids_and_uniform_weights():
    ids, w, _ = ro.route(f16(np.zeros((3, 8))), f16(np.ones((5, 8))), 3)
    assert ids.tolist() == [[0, 1, 2]] * 3
    np.testing.assert_allclose(w, 1 / 3, atol=1e-15)


# --- planted mistakes: each must break one of the pins above --------------
def test_planted_mistakes_are_caught(monkeypatch):
    rng = np.random.default_rng(0)
    x = f16(rng.standard_normal((5, 16)))
    wr = f16(rng.normal(0, 0.5, (7, 16)))
    bi, bw = route_bruteforce(x, wr, 3)
    good = ro.topk_select

    def ascending(logits, k):
        T, E = logits.shape
        return np.array([sorted(range(E), key=lambda e: (logits[t, e], e))[:k] for t in range(T)], np.int32)

    def higher_id_first(logits, k):
        T, E = logits.shape
        return np.array([sorted(range(E), key=lambda e: (-logits[t, e], -e))[:k] for t in range(T)], np.int32)

    def softmax_all(logits, ids):
        z = np.exp(logits - logits.max(axis=1, keepdims=True))
        p = z / z.sum(axis=1, keepdims=True)
        return np.take_along_axis(p, ids.astype(np.int64), axis=1)

    for name, fn in [("topk_select", ascending), ("topk_softmax", softmax_all)]:
        with monkeypatch.context() as m:
            m.setattr(ro, name, fn)
            ids, w, _ = ro.route(x, wr, 3)
            assert not (np.array_equal(ids, bi) and np.allclose(w, bw, atol=1e-12)), name
    # the tie rule is only visible on ties: the hand-worked example pins it
    with monkeypatch.context() as m:
        m.setattr(ro, "topk_select", higher_id_first)
        ids, _, _ = ro.route(f16([[0, 0], [1, 1]]), f16([[0, 1], [1, 0], [2, 0], [-1, 0]]), 2)
        assert ids.tolist() != [[0, 1], [2, 0]]
    assert ro.topk_select is good
