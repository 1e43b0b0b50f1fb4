"""Pins for the oracle's dynamic (confidence-ranked) tree: the N most probable candidate paths.

References: a hand-worked example whose probabilities are powers of two (joint log-probabilities
then tie exactly, so the tie rules are exercised; every path cost is listed below), equal
probabilities (the tree is then the breadth-first prefix of the full tree, a static branching
tree), an independent best-first search with a heap (the classic lazy enumeration: pop the best
path, push its first child and its next sibling), the top-N exchange property, width limits and
taking every path.
"""
import heapq
import math

import numpy as np
import pytest

from oracle import medusa_oracle as O


def _pow2_case():
    # head k's candidate probabilities as powers of two: logits -k*ln2, LSE 0
    # depth 1: 1/2, 1/4, 1/8    depth 2: 1/2, 1/4, 1/4    depth 3: 1/2, 1/2
    ln2 = np.float32(math.log(2.0))
    k = np.array([[[1, 2, 3], [1, 2, 2], [1, 1, 9]]], np.float32)
    vals = -k * ln2
    ids = np.array([[[10, 11, 12], [20, 21, 22], [30, 31, 32]]], np.int32)
    return ids, vals, np.zeros((1, 3), np.float32)


def test_hand_example_with_exact_ties():
    # path costs in units of ln 2 (smaller = more probable):
    #   (0):1  (1):2  (0,0):2  (2):3  (0,1):3  (0,2):3  (1,0):3  (0,0,0):3  (0,0,1):3 ...
    # order: cost, then depth, then ranks -> (0), (1), (0,0), (2), (0,1), (0,2), (1,0), (0,0,0)
    ids, vals, lse = _pow2_case()
    r = O.dynamic_tree(ids, vals, lse, (3, 3, 2), 6)
    assert r["parents"][0] == [-1, -1, -1, 0, 0, 0]
    assert r["tokens"][0] == [10, 11, 12, 20, 21, 22]
    assert r["ranks"][0] == [(0,), (1,), (2,), (0, 0), (0, 1), (0, 2)]
    r = O.dynamic_tree(ids, vals, lse, (3, 3, 2), 8)
    assert r["parents"][0] == [-1, -1, -1, 0, 0, 0, 1, 3]
    assert r["depth"][0] == [1, 1, 1, 2, 2, 2, 2, 3]
    assert r["tokens"][0] == [10, 11, 12, 20, 21, 22, 20, 30]
    ln2 = float(np.float32(math.log(2.0)))
    assert r["score"][0] == [-ln2, -2 * ln2, -3 * ln2, -2 * ln2, -3 * ln2, -3 * ln2,
                             -3 * ln2, -3 * ln2]
    # only 5 nodes: (2) and (0,1) tie at cost 3 and depth decides -> (2) is in, (0,1) out
    r = O.dynamic_tree(ids, vals, lse, (3, 3, 2), 4)
    assert r["ranks"][0] == [(0,), (1,), (2,), (0, 0)]


@pytest.mark.parametrize("s,N,want", [
    ((2, 2, 2), 6, [-1, -1, 0, 0, 1, 1]),
    ((2, 2, 2), 5, [-1, -1, 0, 0, 1]),
    ((3, 2), 9, [-1, -1, -1, 0, 0, 1, 1, 2, 2]),
])
def test_equal_probabilities_give_the_breadth_first_full_tree(s, N, want):
    D = len(s)
    vals = np.zeros((1, D, 4), np.float32)
    ids = np.arange(D * 4, dtype=np.int32).reshape(1, D, 4)
    r = O.dynamic_tree(ids, vals, None, s, N)
    assert r["parents"][0] == want


def _best_first(logp, s, N):
    """Lazy enumeration: a heap of (-score, depth, ranks); popping a path pushes its first
    child and its next sibling."""
    D = len(s)
    heap = [(-logp[0][0], 1, (0,), 0.0)]
    out = []
    while len(out) < N:
        neg, d, rk, parent_score = heapq.heappop(heap)
        out.append((rk, -neg))
        if d < D:
            heapq.heappush(heap, (-(-neg + logp[d][0]), d + 1, rk + (0,), -neg))
        if rk[-1] + 1 < s[d - 1]:
            heapq.heappush(heap, (-(parent_score + logp[d - 1][rk[-1] + 1]), d,
                                  rk[:-1] + (rk[-1] + 1,), parent_score))
    return out


@pytest.mark.parametrize("seed", range(5))
def test_matches_independent_best_first_search(seed):
    rng = np.random.default_rng(seed)
    B, D, smax = 3, 4, 6
    s = (6, 5, 3, 2)
    N = [1, 17, 64][seed % 3]
    logits = rng.standard_normal((B, D, 50)) * 2.0
    top = np.argsort(-logits, axis=2, kind="stable")[:, :, :smax]
    vals = np.take_along_axis(logits, top, axis=2).astype(np.float32)
    lse = np.log(np.exp(logits).sum(axis=2)).astype(np.float32)
    r = O.dynamic_tree(top.astype(np.int32), vals, lse, s, N)
    for b in range(B):
        logp = vals[b].astype(np.float64) - lse[b].astype(np.float64)[:, None]
        bf = _best_first(logp, s, N)
        assert sorted(rk for rk, _ in bf) == sorted(r["ranks"][b])
        sc = dict(bf)
        assert [sc[rk] for rk in r["ranks"][b]] == r["score"][b]     # same fp64 sums
        # layout: breadth first, parents before children, children of a node in rank order
        for i, (p, rk) in enumerate(zip(r["parents"][b], r["ranks"][b])):
            assert p < i
            if p >= 0:
                assert r["ranks"][b][p] == rk[:-1]
            assert r["tokens"][b][i] == top[b, len(rk) - 1, rk[-1]]


def test_top_n_exchange_property():
    """Every path left out whose parent is in the tree (or that is a root) scores no higher
    than every path in the tree."""
    rng = np.random.default_rng(11)
    D, s, N = 3, (5, 4, 4), 20
    vals = -np.sort(rng.exponential(1.0, (1, D, 5)), axis=2).astype(np.float32)
    r = O.dynamic_tree(np.zeros((1, D, 5), np.int32), vals, None, s, N)
    chosen = set(r["ranks"][0])
    worst = min(r["score"][0])
    score = lambda rk: sum(float(vals[0, k, x]) for k, x in enumerate(rk))
    for rk in list(chosen) + [()]:
        d = len(rk)
        if d < D:
            for x in range(s[d]):
                if rk + (x,) not in chosen:
                    assert score(rk + (x,)) <= worst + 1e-12


def test_positive_log_probabilities_count_as_zero():
    """A head whose top candidate has val - lse slightly above 0 (rounding): clamped, so the
    child of a path never outranks it and the result is still a tree."""
    vals = np.array([[[1e-7, -1.0], [2e-7, -0.5]]], np.float32)
    r = O.dynamic_tree(np.zeros((1, 2, 2), np.int32), vals, None, (2, 2), 3)
    assert r["ranks"][0] == [(0,), (0, 0), (0, 1)]
    assert r["score"][0][:2] == [0.0, 0.0]


def test_widths_and_taking_every_path():
    ids = np.arange(24, dtype=np.int32).reshape(1, 3, 8)
    vals = -np.sort(np.random.default_rng(3).exponential(1.0, (1, 3, 8)),
                    axis=2).astype(np.float32)
    s = (2, 3, 1)
    total = 2 + 2 * 3 + 2 * 3 * 1
    r = O.dynamic_tree(ids, vals, None, s, total)
    assert len(r["parents"][0]) == total
    assert max(rk[k] for rk in r["ranks"][0] for k in range(len(rk))) <= 2
    for rk, t in zip(r["ranks"][0], r["tokens"][0]):
        assert rk[-1] < s[len(rk) - 1] and t == ids[0, len(rk) - 1, rk[-1]]
    with pytest.raises(ValueError):
        O.dynamic_tree(ids, vals, None, s, total + 1)
