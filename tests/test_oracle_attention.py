"""Pins for the oracle's tree attention.

References that do not share the oracle's formula:
* brute force: each root-to-leaf path run as its own causal sequence
  (prefix ++ path) through torch's scaled_dot_product_attention;
* a chain tree equals causal attention over prefix + chain;
* a one-node tree equals plain decode attention;
* closed forms: constant V rows, and K = 0 (uniform weights over visible keys).
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import medusa_oracle as O
from medusa_tree_attention_verify_amd.workloads import branching_tree, chain_tree


def _inputs(seed, B, N, Hq, Hkv, dh, lens):
    rng = np.random.default_rng(seed)
    L_cap = max(lens) + N
    q = rng.standard_normal((B, N, Hq, dh))
    k = rng.standard_normal((B, Hkv, L_cap, dh))
    v = rng.standard_normal((B, Hkv, L_cap, dh))
    return q, k, v, np.array(lens, dtype=np.int32)


def _sdpa(q, k, v, mask, scale):
    """q [Hq, Lq, dh], k/v [Hkv, Lk, dh] (fp64 torch), boolean mask [Lq, Lk] or None."""
    return F.scaled_dot_product_attention(
        q.unsqueeze(0), k.unsqueeze(0), v.unsqueeze(0), attn_mask=mask, scale=scale,
        enable_gqa=True).squeeze(0)


@pytest.mark.parametrize("widths,Hq,Hkv", [((3, 2, 2), 4, 2), ((2, 3, 1, 2), 6, 3), ((4, 1), 2, 2)])
def test_brute_force_paths(widths, Hq, Hkv):
    parents = branching_tree(widths)
    N, dh, B = len(parents), 16, 2
    q, k, v, lens = _inputs(1, B, N, Hq, Hkv, dh, [11, 7])
    t = O.build_tree(parents)
    res = O.tree_attention(q, k, v, lens, t["anc"])
    children = {p for p in parents}
    leaves = [i for i in range(N) if i not in children]
    scale = 1 / math.sqrt(dh)
    for b in range(B):
        L = int(lens[b])
        for leaf in leaves:
            path = t["anc"][leaf]                  # root ... leaf, sorted == path order
            rows = list(range(L)) + [L + j for j in path]
            kk = torch.from_numpy(k[b][:, rows])
            vv = torch.from_numpy(v[b][:, rows])
            qq = torch.from_numpy(q[b][path].transpose(1, 0, 2).copy())   # [Hq, len, dh]
            n = len(path)
            causal = torch.ones(n, L + n, dtype=torch.bool)
            causal[:, L:] = torch.tril(torch.ones(n, n, dtype=torch.bool))
            ref = _sdpa(qq, kk, vv, causal, scale).numpy()                   # [Hq, len, dh]
            for pos, node in enumerate(path):
                np.testing.assert_allclose(res["out"][b, node], ref[:, pos], rtol=0, atol=1e-12)


def test_chain_equals_causal():
    N, Hq, Hkv, dh = 9, 4, 1, 32
    q, k, v, lens = _inputs(2, 1, N, Hq, Hkv, dh, [20])
    t = O.build_tree(chain_tree(N))
    res = O.tree_attention(q, k, v, lens, t["anc"])
    L = 20
    qq = torch.from_numpy(q[0].transpose(1, 0, 2).copy())
    kk = torch.from_numpy(k[0][:, :L + N])
    vv = torch.from_numpy(v[0][:, :L + N])
    # bottom-right aligned causal mask: query j sees keys [0, L + j]
    mask = torch.ones(N, L + N, dtype=torch.bool).tril(diagonal=L)
    ref = _sdpa(qq, kk, vv, mask, 1 / math.sqrt(dh)).numpy()
    np.testing.assert_allclose(res["out"][0], ref.transpose(1, 0, 2), rtol=0, atol=1e-12)


def test_single_node_is_decode():
    Hq, Hkv, dh = 8, 2, 64
    q, k, v, lens = _inputs(3, 3, 1, Hq, Hkv, dh, [5, 33, 17])
    t = O.build_tree([-1])
    res = O.tree_attention(q, k, v, lens, t["anc"])
    for b in range(3):
        L = int(lens[b])
        qq = torch.from_numpy(q[b].transpose(1, 0, 2).copy())       # [Hq, 1, dh]
        ref = _sdpa(qq, torch.from_numpy(k[b][:, :L + 1]), torch.from_numpy(v[b][:, :L + 1]),
                    None, 1 / math.sqrt(dh)).numpy()
        np.testing.assert_allclose(res["out"][b], ref.transpose(1, 0, 2), rtol=0, atol=1e-12)


def test_constant_values_and_zero_keys():
    parents = branching_tree((2, 2, 1))
    N, Hq, Hkv, dh = len(parents), 4, 2, 8
    q, k, v, lens = _inputs(4, 1, N, Hq, Hkv, dh, [6])
    t = O.build_tree(parents)
    # constant V rows: every output equals that row, whatever the weights
    c = np.arange(dh, dtype=np.float64)
    v_const = np.broadcast_to(c, v.shape).copy()
    out = O.tree_attention(q, k, v_const, lens, t["anc"])["out"]
    np.testing.assert_allclose(out, np.broadcast_to(c, out.shape), rtol=0, atol=1e-12)
    # K = 0: uniform weights -> mean of the visible V rows; lse = log(count)
    res = O.tree_attention(q, np.zeros_like(k), v, lens, t["anc"])
    L = 6
    for i in range(N):
        rows = list(range(L)) + [L + j for j in t["anc"][i]]
        for h in range(Hq):
            g = h // (Hq // Hkv)
            np.testing.assert_allclose(res["out"][0, i, h], v[0, g, rows].mean(axis=0), atol=1e-12)
            assert abs(res["lse"][0, h, i] - math.log(len(rows))) < 1e-12


def test_masked_tree_keys_have_no_influence():
    # changing the K/V of a node outside i's ancestor set must not change node i
    parents = branching_tree((2, 2))
    N, dh = len(parents), 16
    q, k, v, lens = _inputs(5, 1, N, 2, 1, dh, [4])
    t = O.build_tree(parents)
    a = O.tree_attention(q, k, v, lens, t["anc"])["out"]
    k2, v2 = k.copy(), v.copy()
    L = 4
    k2[0, :, L + 1] += 5.0      # node 1 (a depth-1 node): invisible to node 0 and its subtree
    v2[0, :, L + 1] -= 3.0
    b = O.tree_attention(q, k2, v2, lens, t["anc"])["out"]
    for i in range(N):
        if 1 in t["anc"][i]:
            assert not np.allclose(a[0, i], b[0, i])
        else:
            np.testing.assert_array_equal(a[0, i], b[0, i])


def test_select_subset_matches_full():
    parents = branching_tree((2, 2))
    q, k, v, lens = _inputs(6, 2, len(parents), 4, 2, 8, [3, 9])
    t = O.build_tree(parents)
    full = O.tree_attention(q, k, v, lens, t["anc"])
    sel = [(1, 3, 5), (0, 0, 0), (1, 2, 2)]
    part = O.tree_attention(q, k, v, lens, t["anc"], select=sel)
    for b, h, i in sel:
        np.testing.assert_array_equal(part["out"][b, i, h], full["out"][b, i, h])
        assert part["lse"][b, h, i] == full["lse"][b, h, i]
