"""GPU parity of candidate-tree assembly (mv_build_tree_mask) against the oracle."""
import json
import os

import numpy as np
import pytest
import torch

from oracle import medusa_oracle as O
from medusa_tree_attention_verify_amd import _lib as L
from medusa_tree_attention_verify_amd import ops
from medusa_tree_attention_verify_amd.workloads import branching_tree, chain_tree, two_chains_tree
from tests.gpu_util import dev_i32, host, require_gpu

pytestmark = pytest.mark.gpu


def _bits(anc_i32):
    return host(anc_i32).astype(np.int64).astype(np.uint32)


def _random_tree(rng, N, max_depth=None):
    parents = []
    depth = []
    for i in range(N):
        cands = [-1] + [j for j in range(i) if max_depth is None or depth[j] < max_depth]
        p = int(rng.choice(cands)) if i else -1
        parents.append(p)
        depth.append(1 if p == -1 else depth[p] + 1)
    return parents


def _run(parents, cand=None, widths=None):
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = ops.build_tree_mask(dev_i32(parents), None if cand is None else dev_i32(cand),
                              widths, status=status)
    torch.cuda.synchronize()
    return out, int(status.item())


def test_page_masks(golden_dir):
    require_gpu()
    with open(os.path.join(golden_dir, "p3_mask_example.json")) as f:
        g3 = json.load(f)
    out, st = _run(g3["parents_reading"])
    assert st == 0
    bits = _bits(out["anc_mask"])[:, 0]
    printed = np.array([[c == "0" for c in row] for row in g3["additive_mask"]])
    for i in range(5):
        row = [(int(bits[i]) >> j) & 1 == 1 for j in range(5)]
        assert row == printed[i].tolist()
    with open(os.path.join(golden_dir, "p4_forest.json")) as f:
        g4 = json.load(f)
    out, st = _run(g4["parents"])
    assert st == 0
    bits = _bits(out["anc_mask"])[:, 0]
    for i, want in enumerate(g4["attends_to"]):
        assert [j for j in range(len(g4["parents"])) if (int(bits[i]) >> j) & 1] == want


@pytest.mark.parametrize("kind,N", [("chain", 1), ("chain", 9), ("two_chains", 8),
                                    ("4321", 64), ("4442", 212), ("random", 33),
                                    ("random", 100), ("random", 256)])
def test_tree_matches_oracle(kind, N):
    require_gpu()
    rng = np.random.default_rng(N)
    if kind == "chain":
        parents = chain_tree(N)
    elif kind == "two_chains":
        parents = two_chains_tree()
    elif kind == "4321":
        parents = branching_tree((4, 3, 2, 1))
    elif kind == "4442":
        parents = branching_tree((4, 4, 4, 2))
    else:
        parents = _random_tree(rng, N, max_depth=12)
    N = len(parents)
    ref = O.build_tree(parents)
    D = int(ref["depth"].max())
    s_max = int(ref["rank"].max()) + 1
    B = 3
    cand = rng.integers(0, 50000, size=(B, D, s_max)).astype(np.int32)
    widths = [s_max] * D
    ref = O.build_tree(parents, [cand[:, k] for k in range(D)], widths)
    out, st = _run(parents, cand, widths)
    assert st == 0
    np.testing.assert_array_equal(_bits(out["anc_mask"]), ref["mask_bits"])
    np.testing.assert_array_equal(host(out["depth"]), ref["depth"])
    np.testing.assert_array_equal(host(out["node_tokens"]), ref["tokens"])


def test_invalid_trees_flag_status():
    require_gpu()
    # parent not topological
    _, st = _run([-1, 0, 3, 1])
    assert st & L.MV_DEV_BAD_PARENT
    # rank beyond the width of its depth: three children of the root, width 2 at depth 1
    cand = np.zeros((1, 2, 2), dtype=np.int32)
    _, st = _run([-1, -1, -1, 0], cand, [2, 2])
    assert st & L.MV_DEV_BAD_RANK
    # deeper than D
    cand = np.zeros((1, 2, 1), dtype=np.int32)
    _, st = _run(chain_tree(3), cand, [1, 1])
    assert st & L.MV_DEV_TOO_DEEP
