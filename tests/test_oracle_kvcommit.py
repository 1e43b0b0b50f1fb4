"""Pins for the oracle's commit of the accepted path into the KV cache.

References: hand-labelled caches whose expected rows are written out (the overlapping path
[1, 3]), special cases (the identity path of a chain, an empty path), rejection of paths that
are not root paths of level-ordered nodes, and the property that makes the commit correct:
after it, causal attention over prefix + kept path reproduces the tree attention that the
path's nodes had before it (a node sees its ancestors only), for every node on the path.
"""
import numpy as np
import pytest

from oracle import medusa_oracle as O


def _labelled(B, Hkv, L_cap, dh):
    """Row r of head g of sequence b holds the value 1000 b + 100 g + r (+ column / 1000)."""
    b, g, r, c = np.meshgrid(np.arange(B), np.arange(Hkv), np.arange(L_cap), np.arange(dh),
                             indexing="ij")
    k = 1000.0 * b + 100.0 * g + r + c / 1000.0
    return k, -k


def test_overlapping_path_hand_example():
    # tree: 0 and 1 are roots, 2 under 0, 3 under 1; accepted path 1 -> 3
    k, v = _labelled(2, 2, 12, 4)
    prefix = np.array([5, 3])
    path = np.array([[1, 3, 0], [0, 2, 0]], dtype=np.int32)
    alen = np.array([2, 1])
    k2, v2, p2 = O.kv_commit(k, v, prefix, path, alen, N=4)
    assert p2.tolist() == [7, 4]
    # sequence 0: rows 5, 6 <- rows 6, 8; the rest unchanged
    assert k2[0, 1, 5, 0] == 106.0 and k2[0, 1, 6, 0] == 108.0
    assert k2[0, 0, 5, 2] == 6.002 and v2[0, 0, 6, 3] == -8.003
    np.testing.assert_array_equal(k2[0, :, :5], k[0, :, :5])
    np.testing.assert_array_equal(k2[0, :, 7:], k[0, :, 7:])
    # sequence 1: row 3 <- row 3 (node 0 at level 0)
    np.testing.assert_array_equal(k2[1], k[1])
    np.testing.assert_array_equal(v2[1], v[1])
    # the input is not modified
    assert k[0, 0, 5, 0] == 5.0


def test_chain_identity_and_empty_path():
    k, v = _labelled(2, 1, 10, 2)
    path = np.array([[0, 1, 2], [0, 1, 2]], dtype=np.int32)
    k2, v2, p2 = O.kv_commit(k, v, np.array([4, 2]), path, np.array([3, 0]), N=3)
    np.testing.assert_array_equal(k2, k)
    np.testing.assert_array_equal(v2, v)
    assert p2.tolist() == [7, 2]


@pytest.mark.parametrize("path,alen,prefix", [
    ([0, 0], 2, 3),     # node 0 on level 1: a node on level j has index >= j
    ([0, 5], 2, 3),     # node outside [0, N)
    ([0, 1], 3, 3),     # length beyond D
    ([0, 1], -1, 3),    # negative length
    ([0, 1], 1, 8),     # tree block [8, 13) beyond L_cap = 12
])
def test_invalid_paths_rejected(path, alen, prefix):
    k, v = _labelled(1, 1, 12, 2)
    with pytest.raises(ValueError):
        O.kv_commit(k, v, np.array([prefix]), np.array([path]), np.array([alen]), N=5)


def test_tree_block_ending_at_capacity_is_valid():
    k, v = _labelled(1, 1, 12, 2)
    k2, _, p2 = O.kv_commit(k, v, np.array([7]), np.array([[4, 1]]), np.array([1]), N=5)
    assert p2.tolist() == [8] and k2[0, 0, 7, 0] == 11.0


def test_commit_turns_tree_attention_into_causal_attention():
    """Before the commit, node path[j] attends to the prefix and its ancestors path[0..j];
    after it, the same query at position L + j attends causally to rows [0, L + j].  Both
    views must give the same output and LSE for every node on the path."""
    rng = np.random.default_rng(7)
    parents = [-1, -1, 0, 0, 1, 2, 2, 3, 4, 5, 6]
    N, B, Hq, Hkv, dh, L_cap = len(parents), 2, 4, 2, 8, 40
    anc = O.build_tree(parents)["anc"]
    prefix = np.array([9, 17])
    q = rng.standard_normal((B, N, Hq, dh))
    k = rng.standard_normal((B, Hkv, L_cap, dh))
    v = rng.standard_normal((B, Hkv, L_cap, dh))
    paths = [[0, 2, 5, 9], [1, 4, 8]]
    D = 4
    path_nodes = np.zeros((B, D), dtype=np.int32)
    for b, p in enumerate(paths):
        path_nodes[b, :len(p)] = p
    alen = np.array([len(p) for p in paths])
    pre = O.tree_attention(q, k, v, prefix, anc)
    k2, v2, p2 = O.kv_commit(k, v, prefix, path_nodes, alen, N)
    assert p2.tolist() == [9 + 4, 17 + 3]
    for b, p in enumerate(paths):
        L = int(prefix[b])
        for j, node in enumerate(p):
            # plain causal softmax over rows [0, L + j] of the committed cache
            for h in range(Hq):
                g = h // (Hq // Hkv)
                s = k2[b, g, :L + j + 1] @ q[b, node, h] / np.sqrt(dh)
                e = np.exp(s - s.max())
                out = e @ v2[b, g, :L + j + 1] / e.sum()
                np.testing.assert_allclose(out, pre["out"][b, node, h], rtol=0, atol=1e-12)
                np.testing.assert_allclose(s.max() + np.log(e.sum()), pre["lse"][b, h, node],
                                           rtol=0, atol=1e-12)
    # the kept path also matches a chain tree over the committed rows
    chain = [list(range(j + 1)) for j in range(D)]
    qc = np.zeros((B, D, Hq, dh))
    for b, p in enumerate(paths):
        qc[b, :len(p)] = q[b, p]
    post = O.tree_attention(qc, k2, v2, prefix, chain)
    for b, p in enumerate(paths):
        np.testing.assert_allclose(post["out"][b, :len(p)], pre["out"][b, p], atol=1e-12)
