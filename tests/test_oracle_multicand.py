"""Pins for the oracle's multi-candidate (sibling-recursive) speculative acceptance.

References: two hand-worked trees of three sibling candidates over a 4-token vocabulary (every
alpha, residual and draw computed by hand below), the single-candidate rule on chains (one
child per node: the recursive rule must make exactly the decisions and draws of the pages'
rule), P_d = P_t (every first candidate is accepted), and chi-square tests of losslessness:
with candidates drawn independently from the parent row's P_d, the first emitted token follows
P_t of the prefix row and the second follows P_t of the first token's row, on branching trees.
"""
import numpy as np
import pytest
from scipy.stats import chisquare

from oracle import medusa_oracle as O

P0 = [0.4, 0.3, 0.2, 0.1]
Q0 = [0.1, 0.5, 0.1, 0.3]


def _three_roots(tokens, u, leaf_row):
    # three root candidates (no deeper nodes); rows 1..3 belong to the roots
    p_t = np.array([[P0, leaf_row, leaf_row, leaf_row]])
    p_d = np.array([[Q0, Q0, Q0, Q0]])
    return O.accept_multicandidate(p_t, p_d, np.array([tokens]), [-1, -1, -1],
                                   np.array([u]), D=1)


def test_hand_example_residual_lowers_alpha():
    # node 0 (token 1): alpha = 0.3/0.5 = 0.6, u = 0.8 rejects;
    #   P1 = normalize(max(0, P0 - Q0)) = normalize([0.3, 0, 0.1, 0]) = [0.75, 0, 0.25, 0]
    # node 1 (token 3): alpha = P1[3]/0.3 = 0 (the plain rule would give 1/3); u = 0.2 rejects;
    #   P2 = normalize(max(0, P1 - Q0)) = normalize([0.65, 0, 0.15, 0]) = [0.8125, 0, 0.1875, 0]
    # node 2 (token 2): alpha = min(1, 0.1875/0.1) = 1, accepted; a leaf, so the extra token
    #   comes from its own row [0.1, 0.6, 0.3, 0] with u = 0.65: cumsum 0.1, 0.7 -> token 1
    r = _three_roots([1, 3, 2], [0.8, 0.2, 0.95, 0.65], [0.1, 0.6, 0.3, 0.0])
    np.testing.assert_allclose(r["alpha"][0], [0.6, 0.0, 1.0], rtol=1e-15)
    assert r["accept_len"].tolist() == [1]
    assert r["path_nodes"][0].tolist() == [2]
    assert r["out_tokens"][0].tolist() == [2, 1]
    assert r["node_accept"][0].tolist() == [False, False, True]


def test_hand_example_all_rejected_draws_from_recursive_residual():
    # as above up to P2 = [0.8125, 0, 0.1875, 0]; node 2 (token 1): alpha = 0, u = 0.95
    # rejects; P3 = normalize(max(0, P2 - Q0)) = normalize([0.7125, 0, 0.0875, 0])
    #   = [0.890625, 0, 0.109375, 0]; u = 0.9 > 0.890625 -> token 2
    r = _three_roots([1, 3, 1], [0.8, 0.2, 0.95, 0.9], [0.25, 0.25, 0.25, 0.25])
    np.testing.assert_allclose(r["alpha"][0], [0.6, 0.0, 0.0], rtol=1e-15)
    assert r["accept_len"].tolist() == [0]
    assert r["out_tokens"][0].tolist() == [2, -1]
    # with u = 0.89 the same residual gives token 0
    r = _three_roots([1, 3, 1], [0.8, 0.2, 0.95, 0.89], [0.25, 0.25, 0.25, 0.25])
    assert r["out_tokens"][0].tolist() == [0, -1]


def test_untested_nodes_and_deeper_walk():
    # tree: 0, 1 roots; 2, 3 under 0; 4 under 1.  Node 0 accepted (P_d = P_t), node 2
    # accepted, so nodes 1, 3, 4 are never tested
    V = 3
    rng = np.random.default_rng(0)
    p = rng.dirichlet(np.ones(V), size=(1, 6))
    parents = [-1, -1, 0, 0, 1]
    r = O.accept_multicandidate(p, p, np.array([[0, 1, 2, 0, 1]]), parents,
                                np.array([[0.5, 0.5, 0.5, 0.5, 0.5, 0.3]]), D=2)
    assert r["path_nodes"][0].tolist() == [0, 2]
    np.testing.assert_array_equal(r["alpha"][0], [1.0, -1.0, 1.0, -1.0, -1.0])
    # extra token from node 2's row (a leaf)
    c = np.cumsum(p[0, 3])
    assert r["out_tokens"][0, 2] == int(np.nonzero(c > 0.3 * c[-1])[0][0])


@pytest.mark.parametrize("seed", range(6))
def test_chains_match_single_candidate_rule(seed):
    """One child per node: the recursive rule never tests a second sibling, so its decisions,
    path and extra token are exactly those of the single-candidate rule."""
    rng = np.random.default_rng(seed)
    B, N, V = 8, 6, 11
    parents = [-1] + list(range(N - 1))
    p_t = rng.dirichlet(np.ones(V), size=(B, N + 1))
    p_d = rng.dirichlet(np.ones(V), size=(B, N + 1))
    toks = rng.integers(0, V, (B, N))
    u = rng.random((B, N + 1))
    a = O.accept_multicandidate(p_t, p_d, toks, parents, u, N)
    s = O.accept_speculative(p_t, p_d, toks, parents, u, N)
    for k in ("accept_len", "path_nodes", "out_tokens"):
        np.testing.assert_array_equal(a[k], s[k], err_msg=k)
    np.testing.assert_array_equal(a["node_accept"], s["node_accept"])
    tested = a["alpha"] >= 0
    np.testing.assert_allclose(a["alpha"][tested], s["alpha"][tested], rtol=1e-15)
    # tested = the path plus the first rejected node below it (if any)
    assert np.all(tested.sum(axis=1) == np.minimum(a["accept_len"] + 1, N))


def _token_tree(width1, width2):
    parents = [-1] * width1
    for i in range(width1):
        parents += [i] * width2
    return parents


def test_lossless_first_and_second_token_chi_square():
    """Candidates drawn independently from the parent row's P_d on a (3, 2) tree; the target
    rows depend only on the token path.  Over 30000 trials the first emitted token follows
    P_t of the prefix row and, given the first token a with the path accepted past it, the
    second follows P_t of a's row."""
    rng = np.random.default_rng(123)
    V, T = 5, 30000
    parents = _token_tree(3, 2)
    N = len(parents)
    pt0 = rng.dirichlet(np.ones(V))
    pd0 = rng.dirichlet(np.ones(V))
    pt1 = rng.dirichlet(np.ones(V), size=V)      # target after token a
    pd1 = rng.dirichlet(np.ones(V), size=V)      # draft after token a
    pt2 = rng.dirichlet(np.ones(V), size=(V, V))  # target after tokens a, b
    pd2 = np.full((V, V, V), 1.0 / V)
    first = np.zeros(V)
    second = np.zeros((V, V))
    for _ in range(T):
        toks = np.zeros(N, dtype=np.int64)
        toks[:3] = rng.choice(V, size=3, p=pd0)
        for i in range(3):
            kids = [3 + 2 * i, 4 + 2 * i]
            toks[kids] = rng.choice(V, size=2, p=pd1[toks[i]])
        p_t = np.empty((1, N + 1, V))
        p_d = np.empty((1, N + 1, V))
        p_t[0, 0], p_d[0, 0] = pt0, pd0
        for i in range(N):
            if parents[i] == -1:
                p_t[0, i + 1], p_d[0, i + 1] = pt1[toks[i]], pd1[toks[i]]
            else:
                a = toks[parents[i]]
                p_t[0, i + 1], p_d[0, i + 1] = pt2[a, toks[i]], pd2[a, toks[i]]
        r = O.accept_multicandidate(p_t, p_d, toks[None], parents, rng.random((1, N + 1)), 2)
        out = r["out_tokens"][0]
        first[out[0]] += 1
        if r["accept_len"][0] >= 1:
            second[out[0], out[1]] += 1
    assert chisquare(first, pt0 * T).pvalue > 1e-3
    for a in range(V):
        n = second[a].sum()
        if n >= 500:
            assert chisquare(second[a], pt1[a] * n).pvalue > 1e-3, a


def test_single_candidate_rule_is_lossy_on_the_same_tree():
    """Control for the chi-square above: the node-by-node rule (every node tested on its own
    against P_t / P_d, extra token from the terminal's residual) does not preserve P_t when a
    node has several candidates; the same test detects it."""
    rng = np.random.default_rng(7)
    V, T = 5, 30000
    parents = [-1, -1, -1]
    pt0 = np.array([0.05, 0.05, 0.1, 0.2, 0.6])
    pd0 = np.array([0.6, 0.2, 0.1, 0.05, 0.05])
    leaf = np.full(V, 1.0 / V)
    p_t = np.array([[pt0, leaf, leaf, leaf]])
    p_d = np.array([[pd0, leaf, leaf, leaf]])
    first_multi = np.zeros(V)
    first_single = np.zeros(V)
    for _ in range(T):
        toks = rng.choice(V, size=(1, 3), p=pd0)
        u = rng.random((1, 4))
        first_multi[O.accept_multicandidate(p_t, p_d, toks, parents, u, 1)["out_tokens"][0, 0]] += 1
        first_single[O.accept_speculative(p_t, p_d, toks, parents, u, 1)["out_tokens"][0, 0]] += 1
    assert chisquare(first_multi, pt0 * T).pvalue > 1e-3
    assert chisquare(first_single, pt0 * T).pvalue < 1e-6
