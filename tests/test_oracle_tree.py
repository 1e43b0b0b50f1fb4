"""Pins for the oracle's tree assembly (parents -> depth, rank, ancestor masks, tokens)."""
import json
import os

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from oracle import medusa_oracle as O
from medusa_tree_attention_verify_amd.workloads import branching_tree, chain_tree


def _load(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


def test_p3_printed_five_node_mask(golden_dir):
    g = _load(golden_dir, "p3_mask_example.json")
    t = O.build_tree(g["parents_reading"])
    printed = np.array([[c == "0" for c in row] for row in g["additive_mask"]])
    assert np.array_equal(O.mask_matrix(t["anc"]), printed)


def test_p4_forest_rows(golden_dir):
    g = _load(golden_dir, "p4_forest.json")
    t = O.build_tree(g["parents"])
    assert [list(a) for a in t["anc"]] == g["attends_to"]
    # two roots -> depth 1 for both
    assert list(t["depth"]) == [1, 2, 3, 3, 2, 1, 2]


def test_p3_path_demo_conversion(golden_dir):
    g = _load(golden_dir, "p3_paths_demo.json")
    labels, parents = O.paths_to_parents(g["paths"])
    assert labels == g["expected_labels"]
    assert parents == g["expected_parents"]
    t = O.build_tree(parents)
    assert O.mask_matrix(t["anc"]).shape == tuple(g["expected_mask_shape"])
    # the same shape as the first five nodes of the second page's forest
    forest = _load(golden_dir, "p4_forest.json")
    assert parents == forest["parents"][:5]


def test_branching_counts():
    t = branching_tree((4, 3, 2, 1))
    assert len(t) == 64
    d = O.build_tree(t)["depth"]
    assert [int((d == k).sum()) for k in (1, 2, 3, 4)] == [4, 12, 24, 24]
    assert int(d.sum()) == 196
    t2 = branching_tree((4, 4, 4, 2))
    d2 = O.build_tree(t2)["depth"]
    assert len(t2) == 212 and [int((d2 == k).sum()) for k in (1, 2, 3, 4)] == [4, 16, 64, 128]
    assert int(d2.sum()) == 740


def test_bitmask_layout_word_and_bit():
    # node 40 in the (4,3,2,1) tree: depth 4, ancestors 16+? -> check words directly
    parents = branching_tree((4, 3, 2, 1))
    t = O.build_tree(parents)
    bits = t["mask_bits"]
    assert bits.shape == (64, 2) and bits.dtype == np.uint32
    for i in range(64):
        got = [j for j in range(64) if (int(bits[i, j // 32]) >> (j % 32)) & 1]
        assert got == t["anc"][i]
    # explicit: node 40's chain is 0 -> 4 -> 16 -> 40
    assert t["anc"][40] == [0, 4, 16, 40]
    assert int(bits[40, 0]) == (1 << 0) | (1 << 4) | (1 << 16)
    assert int(bits[40, 1]) == 1 << (40 - 32)


def test_rank_and_tokens_by_hand():
    # root with 3 children; the second child has 2 children
    parents = [-1, 0, 0, 0, 2, 2]
    cand = [np.array([[7]]), np.array([[10, 11, 12]]), np.array([[20, 21]])]
    t = O.build_tree(parents, cand, widths=[1, 3, 2])
    assert list(t["rank"]) == [0, 0, 1, 2, 0, 1]
    assert t["tokens"].tolist() == [[7, 10, 11, 12, 20, 21]]


def test_invalid_trees_rejected():
    with pytest.raises(ValueError):
        O.build_tree([0])              # self parent
    with pytest.raises(ValueError):
        O.build_tree([-1, 2, 0])       # forward reference
    with pytest.raises(ValueError):
        O.build_tree([-2])
    with pytest.raises(ValueError):     # rank beyond the width at depth 1
        O.build_tree([-1, -1], [np.array([[1, 2]])], widths=[1])


def test_chain_is_causal():
    t = O.build_tree(chain_tree(10))
    m = O.mask_matrix(t["anc"])
    assert np.array_equal(m, np.tril(np.ones((10, 10), dtype=bool)))


@st.composite
def random_parents(draw):
    n = draw(st.integers(1, 70))
    return [draw(st.integers(-1, i - 1)) for i in range(n)]


@settings(max_examples=60, deadline=None)
@given(random_parents())
def test_invariants_random_trees(parents):
    t = O.build_tree(parents)
    m = O.mask_matrix(t["anc"])
    n = len(parents)
    assert np.all(np.diag(m))
    assert not np.any(np.triu(m, 1))                 # only earlier (or self) nodes
    for i, p in enumerate(parents):
        assert m[i].sum() == t["depth"][i]
        if p >= 0:
            assert np.all(m[i] >= m[p])                 # parent's set is a subset
            assert m[i].sum() == m[p].sum() + 1
        # walk (the second page's loop) gives the same set
        walk, c = set(), i
        while c != -1:
            walk.add(c)
            c = parents[c]
        assert walk == set(np.nonzero(m[i])[0].tolist())
    assert t["mask_bits"].shape == (n, (n + 31) // 32)
