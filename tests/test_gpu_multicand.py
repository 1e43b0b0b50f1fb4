"""GPU parity of multi-candidate (sibling-recursive) speculative acceptance
(mv_accept_paths(MV_ACCEPT_MULTICAND)) against the oracle, and its losslessness on the GPU."""
import numpy as np
import pytest
import torch
from scipy.stats import chisquare

from oracle import medusa_oracle as O
from medusa_tree_attention_verify_amd import _lib as L
from medusa_tree_attention_verify_amd import ops
from medusa_tree_attention_verify_amd import workloads as W
from medusa_tree_attention_verify_amd.workloads import branching_tree, chain_tree
from tests.gpu_util import dev, dev_i32, host, require_gpu

pytestmark = pytest.mark.gpu


def _run(parents, x, D):
    return ops.accept_paths(L.MV_ACCEPT_MULTICAND, dev_i32(parents), dev_i32(x["node_tokens"]),
                            dev(x["p_target"]), D, draft=dev(x["p_draft"]),
                            uniforms=dev(x["uniforms"]))


def _check(got, x, parents, D, rows=None):
    """Per sequence: outputs exact and alpha within 1e-6 (-1 exactly where untested), except
    sequences where a tested node has |u - alpha| < 1e-6 (counted, skipped)."""
    g = {k: host(v) for k, v in got.items() if v is not None}
    B = x["p_target"].shape[0]
    rows = range(B) if rows is None else rows
    N = len(parents)
    skipped = 0
    for b in rows:
        sl = slice(b, b + 1)
        ref = O.accept_multicandidate(x["p_target"][sl], x["p_draft"][sl], x["node_tokens"][sl],
                                      parents, x["uniforms"][sl], D)
        a = ref["alpha"][0]
        u = x["uniforms"][b, :N].astype(np.float64)
        if np.any((a >= 0) & (np.abs(u - a) < 1e-6)):
            skipped += 1
            continue
        for key in ("accept_len", "path_nodes", "out_tokens"):
            np.testing.assert_array_equal(g[key][b], ref[key][0], err_msg=f"{key} b={b}")
        np.testing.assert_array_equal(g["node_accept"][b].astype(bool), ref["node_accept"][0])
        tested = a >= 0
        np.testing.assert_array_equal(g["alpha"][b][~tested], -1.0)
        assert np.all(np.abs(g["alpha"][b][tested] - a[tested]) <= 1e-6), b
    if skipped:
        print(f"near-tie sequences skipped: {skipped}")
    return skipped


@pytest.mark.parametrize("tree,B,V,noise", [
    ((4, 3, 2, 1), 16, 4096, 1.0),
    ((4, 3, 2, 1), 16, 999, 3.0),        # ragged vocabulary (scalar loads), many rejections
    ((4, 4, 4, 2), 8, 5000, 2.0),
    ((8, 2), 32, 1000, 4.0),             # wide first level: up to 7 residual passes per node
    ("chain", 8, 777, 1.0),
])
def test_multicand_small(tree, B, V, noise):
    require_gpu()
    parents = chain_tree(6) if tree == "chain" else branching_tree(tree)
    D = int(O.build_tree(parents)["depth"].max())
    wl = W.WORKLOADS["c7"].scaled(B=B, parents=tuple(parents), depth_widths=(1,) * D,
                                  accept_V=V, draft_noise_std=noise)
    print(f"multicand tree={tree} B={B} V={V} noise={noise}", flush=True)
    x = W.gen_speculative(wl, 31 + B)
    got = _run(parents, x, D)
    torch.cuda.synchronize()
    assert _check(got, x, parents, D) <= 1
    lens = host(got["accept_len"])
    print("accept lengths", lens.tolist())


def test_multicand_serving_full_sampled():
    """64 sequences, 64-node (4,3,2,1) tree, vocabulary 128256, four/three/two/one independent
    draft samples per node: the GPU decides every sequence, the oracle recomputes 8 sampled
    sequences from their own slices."""
    require_gpu()
    wl = W.WORKLOADS["c7"]
    parents = list(wl.parents)
    print(f"multicand full B={wl.B} V={wl.accept_V}", flush=True)
    x = W.gen_speculative(wl, 19)
    got = _run(parents, x, wl.D)
    torch.cuda.synchronize()
    assert _check(got, x, parents, wl.D, rows=(0, 9, 17, 26, 35, 44, 53, 63)) <= 1


def test_multicand_hand_examples():
    """The hand-worked three-candidate examples over a 4-token vocabulary (the oracle pins):
    a residual that lowers alpha to 0, then acceptance; and all three rejected."""
    require_gpu()
    P0, Q0 = [0.4, 0.3, 0.2, 0.1], [0.1, 0.5, 0.1, 0.3]
    for toks, u, leaf, want_alpha, want_out in (
            ([1, 3, 2], [0.8, 0.2, 0.95, 0.65], [0.1, 0.6, 0.3, 0.0], [0.6, 0.0, 1.0], [2, 1]),
            ([1, 3, 1], [0.8, 0.2, 0.95, 0.9], [0.25] * 4, [0.6, 0.0, 0.0], [2, -1]),
            ([1, 3, 1], [0.8, 0.2, 0.95, 0.89], [0.25] * 4, [0.6, 0.0, 0.0], [0, -1])):
        x = {"p_target": np.array([[P0, leaf, leaf, leaf]], np.float32),
             "p_draft": np.array([[Q0] * 4], np.float32),
             "node_tokens": np.array([toks], np.int32), "uniforms": np.array([u], np.float32)}
        got = _run([-1, -1, -1], x, 1)
        torch.cuda.synchronize()
        np.testing.assert_allclose(host(got["alpha"])[0], want_alpha, atol=1e-6)
        assert host(got["out_tokens"])[0].tolist() == want_out
        _check(got, x, [-1, -1, -1], 1)


def test_multicand_edge_cases():
    require_gpu()
    V = 6
    # a residual that is all zero after a rejection (P_t <= P_d) falls back to P_t
    pt = np.array([0.25, 0.25, 0.0, 0.0, 0.0, 0.0], np.float32)
    pd = np.array([0.5, 0.5, 0.0, 0.0, 0.0, 0.0], np.float32)
    parents = [-1, -1, 0]
    x = {"p_target": np.tile(pt, (1, 4, 1)), "p_draft": np.tile(pd, (1, 4, 1)),
         "node_tokens": np.array([[0, 1, 2]], np.int32),
         "uniforms": np.array([[0.9, 0.9, 0.5, 0.3]], np.float32)}
    got = _run(parents, x, 2)
    torch.cuda.synchronize()
    _check(got, x, parents, 2)
    # P_d(x) = 0 -> alpha = 1; a leaf reached -> extra token from its own row
    x2 = {"p_target": np.tile(np.array([0.1, 0.2, 0.3, 0.4, 0, 0], np.float32), (1, 4, 1)),
          "p_draft": np.tile(np.array([0.5, 0, 0, 0.5, 0, 0], np.float32), (1, 4, 1)),
          "node_tokens": np.array([[1, 2, 3]], np.int32),
          "uniforms": np.array([[0.999, 0.1, 0.5, 0.7]], np.float32)}
    got = _run(parents, x2, 2)
    torch.cuda.synchronize()
    _check(got, x2, parents, 2)
    assert host(got["path_nodes"])[0].tolist() == [0, 2]
    assert host(got["out_tokens"])[0].tolist() == [1, 3, 3]
    # a token outside the vocabulary (node 0, tested first): flagged, that candidate rejected
    # without a residual step, node 1 (P_d = 0 at its token) then accepted
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    x3 = dict(x2, node_tokens=np.array([[9, 2, 3]], np.int32))
    ops.accept_paths(L.MV_ACCEPT_MULTICAND, dev_i32(parents), dev_i32(x3["node_tokens"]),
                     dev(x3["p_target"]), 2, draft=dev(x3["p_draft"]),
                     uniforms=dev(x3["uniforms"]), status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == L.MV_DEV_BAD_TOKEN


def test_multicand_lossless_chi_square_on_gpu():
    """100000 sequences on a (3, 2) tree whose candidates are independent draws from the
    parent row's P_d and whose target rows depend only on the token path: the first emitted
    token follows P_t of the prefix row, and the second (when the walk went past the first
    level) follows P_t of the first token's row.  2000 sequences also against the oracle."""
    require_gpu()
    rng = np.random.default_rng(2024)
    V, T = 8, 100_000
    parents = [-1, -1, -1, 0, 0, 1, 1, 2, 2]
    N = len(parents)
    pt0 = rng.dirichlet(np.ones(V))
    pd0 = rng.dirichlet(np.ones(V) * 0.7)
    pt1 = rng.dirichlet(np.ones(V), size=V)
    pd1 = rng.dirichlet(np.ones(V) * 0.7, size=V)
    pt2 = rng.dirichlet(np.ones(V), size=(V, V))
    pd2 = rng.dirichlet(np.ones(V), size=(V, V))
    t1 = rng.choice(V, size=(T, 3), p=pd0)
    cdf1 = np.cumsum(pd1, axis=1)
    u2 = rng.random((T, 3, 2)) * cdf1[t1][:, :, -1:]
    t2 = np.minimum((u2[..., None] >= cdf1[t1][:, :, None, :]).sum(-1), V - 1)
    toks = np.concatenate([t1, t2.reshape(T, 6)], axis=1).astype(np.int32)
    p_t = np.empty((T, N + 1, V), np.float32)
    p_d = np.empty((T, N + 1, V), np.float32)
    p_t[:, 0], p_d[:, 0] = pt0, pd0
    for i in range(N):
        if parents[i] == -1:
            p_t[:, i + 1], p_d[:, i + 1] = pt1[toks[:, i]], pd1[toks[:, i]]
        else:
            a = toks[:, parents[i]]
            p_t[:, i + 1], p_d[:, i + 1] = pt2[a, toks[:, i]], pd2[a, toks[:, i]]
    u = rng.random((T, N + 1), dtype=np.float32)
    x = {"p_target": p_t, "p_draft": p_d, "node_tokens": toks, "uniforms": u}
    got = _run(parents, x, 2)
    torch.cuda.synchronize()
    out = host(got["out_tokens"])
    alen = host(got["accept_len"])
    # targets as the GPU sees them: the fp32 rows, normalised
    q0 = p_t[0, 0].astype(np.float64) / p_t[0, 0].astype(np.float64).sum()
    assert chisquare(np.bincount(out[:, 0], minlength=V), q0 * T).pvalue > 1e-3
    for a in range(V):
        m = (alen >= 1) & (out[:, 0] == a)
        if m.sum() >= 1000:
            q1 = pt1[a].astype(np.float32).astype(np.float64)
            q1 /= q1.sum()
            assert chisquare(np.bincount(out[m, 1], minlength=V), q1 * m.sum()).pvalue > 1e-3, a
    print("mean accepted length", float(alen.mean()))
    sub = {k: v[:2000] for k, v in x.items()}
    sub_got = {k: (v[:2000] if v is not None else None) for k, v in got.items()}
    _check(sub_got, sub, parents, 2)
