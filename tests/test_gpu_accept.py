"""GPU parity of acceptance (mv_accept_paths): greedy and speculative, against the oracle."""
import json
import os

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


def _tokens(rng, parents, B, V):
    """Distinct tokens among the children of every parent."""
    toks = np.zeros((B, len(parents)), dtype=np.int32)
    for par, kids in W.children_of(parents).items():
        for b in range(B):
            toks[b, kids] = rng.choice(V, size=len(kids), replace=False)
    return toks


def _compare(got, ref, B, D, what):
    np.testing.assert_array_equal(host(got["accept_len"]), ref["accept_len"], err_msg=what)
    np.testing.assert_array_equal(host(got["path_nodes"]), ref["path_nodes"], err_msg=what)
    np.testing.assert_array_equal(host(got["out_tokens"]), ref["out_tokens"], err_msg=what)
    np.testing.assert_array_equal(host(got["node_accept"]).astype(bool), ref["node_accept"],
                                  err_msg=what)


@pytest.mark.parametrize("parents,B,V,dtype,p", [
    (W.two_chains_tree(), 1, 1000, torch.float32, 0.0),
    (W.two_chains_tree(), 64, 1000, torch.float32, 0.7),
    (branching_tree((4, 3, 2, 1)), 1, 32000, torch.bfloat16, 0.6),
    (branching_tree((4, 3, 2, 1)), 8, 32000, torch.bfloat16, 0.6),
    (branching_tree((4, 3, 2, 1)), 300, 999, torch.bfloat16, 0.8),     # ragged vocab
    (branching_tree((4, 4, 4, 2)), 4, 5000, torch.float32, 0.9),
    (chain_tree(6), 50, 64, torch.float32, 0.95),
])
def test_greedy_matches_oracle(parents, B, V, dtype, p):
    require_gpu()
    print(f"greedy N={len(parents)} B={B} V={V} {dtype} p={p}", flush=True)
    rng = np.random.default_rng(B + V)
    D = int(O.build_tree(parents)["depth"].max())
    toks = _tokens(rng, parents, B, V)
    wl = W.Workload(name="g", dtype="f32", B=B, Hq=1, Hkv=1, dh=64, parents=tuple(parents),
                    prefix=(0, 0), depth_widths=(1,) * D, accept_V=V, target_std=2.0)
    logits = W.gen_target_logits(wl, seed=B)
    logits = W.plant_greedy(logits, parents, toks, seed=V, p=p)
    if dtype == torch.bfloat16:
        logits = W.round_bf16(logits)
    got = ops.accept_paths(L.MV_ACCEPT_GREEDY, dev_i32(parents), dev_i32(toks),
                           dev(logits, dtype), D)
    torch.cuda.synchronize()
    ref = O.accept_greedy(logits, toks, parents, D)
    _compare(got, ref, B, D, "greedy")


def _p4_rows(g, V=16):
    parents, probs = g["parents"], g["probs"]
    N = len(parents)
    p_t = np.zeros((1, N + 1, V), dtype=np.float32)
    p_d = np.zeros((1, N + 1, V), dtype=np.float32)
    for i, par in enumerate(parents):
        p_d[0, par + 1, i + 1] = 0.1
        p_t[0, par + 1, i + 1] = np.float32(0.1 * probs[i])
    p_t[:, :, 0] += 0.05
    p_d[:, :, 0] += 0.05
    return p_t, p_d, np.arange(1, N + 1, dtype=np.int32)[None]


def test_speculative_page_demo(golden_dir):
    require_gpu()
    with open(os.path.join(golden_dir, "p4_verify_demo.json")) as f:
        g = json.load(f)
    p_t, p_d, toks = _p4_rows(g)
    N = len(g["parents"])
    u = np.full((1, N + 1), g["threshold"], dtype=np.float32)
    got = ops.accept_paths(L.MV_ACCEPT_SPECULATIVE, dev_i32(g["parents"]), dev_i32(toks),
                           dev(p_t), 4, draft=dev(p_d), uniforms=dev(u))
    torch.cuda.synchronize()
    assert host(got["node_accept"])[0].tolist() == g["expected_accepted_flags"]
    assert host(got["path_nodes"])[0, :3].tolist() == g["expected_path"]
    assert int(host(got["accept_len"])[0]) == g["expected_count"]
    ref = O.accept_speculative(p_t, p_d, toks, g["parents"], u, D=4)
    _compare(got, ref, 1, 4, "p4 demo")


def _spec_case(wl, seed):
    x = W.gen_speculative(wl, seed)
    D = wl.D
    parents = list(wl.parents)
    got = ops.accept_paths(L.MV_ACCEPT_SPECULATIVE, dev_i32(parents), dev_i32(x["node_tokens"]),
                           dev(x["p_target"]), D, draft=dev(x["p_draft"]),
                           uniforms=dev(x["uniforms"]))
    torch.cuda.synchronize()
    ref = O.accept_speculative(x["p_target"], x["p_draft"], x["node_tokens"], parents,
                               x["uniforms"], D)
    # decisions: exact except |u - alpha| < 1e-6 (counted); none is expected
    u = x["uniforms"][:, :wl.N].astype(np.float64)
    near = np.abs(u - ref["alpha"]) < 1e-6
    dec_gpu = host(got["node_accept"]).astype(bool)
    assert np.all(np.abs(host(got["alpha"]) - ref["alpha"]) <= 1e-6)
    if near.any():
        print(f"near-tie decisions: {int(near.sum())}")
    if not near.any():
        _compare(got, ref, wl.B, D, "speculative")
    else:
        ok = ~near.any(axis=1)
        for k in ("accept_len", "path_nodes", "out_tokens"):
            np.testing.assert_array_equal(host(got[k])[ok], ref[k][ok])
    return host(got["accept_len"])


def test_speculative_serving_shape_full_vocab():
    """64-node (4,3,2,1) tree, vocabulary 128256, 16 sequences."""
    require_gpu()
    wl = W.WORKLOADS["c5"].scaled(B=16)
    print("spec B=16 V=128256", flush=True)
    lens = _spec_case(wl, 5)
    print("accept lengths", lens.tolist())


def test_speculative_serving_full_sampled():
    """The full batched-serving acceptance shape (64 sequences, vocabulary 128256): the GPU
    decides every sequence; the oracle recomputes 8 sampled sequences from their own slices of
    the same inputs (acceptance is independent per sequence)."""
    require_gpu()
    wl = W.WORKLOADS["c5"]
    x = W.gen_speculative(wl, 17)
    D, parents = wl.D, list(wl.parents)
    print(f"spec full B={wl.B} V={wl.accept_V}", flush=True)
    got = ops.accept_paths(L.MV_ACCEPT_SPECULATIVE, dev_i32(parents), dev_i32(x["node_tokens"]),
                           dev(x["p_target"]), D, draft=dev(x["p_draft"]),
                           uniforms=dev(x["uniforms"]))
    torch.cuda.synchronize()
    g = {k: host(v) for k, v in got.items() if v is not None}
    for b in (0, 9, 17, 26, 35, 44, 53, 63):
        sl = slice(b, b + 1)
        ref = O.accept_speculative(x["p_target"][sl], x["p_draft"][sl], x["node_tokens"][sl], parents,
                                   x["uniforms"][sl], D)
        u = x["uniforms"][b, :wl.N].astype(np.float64)
        assert np.all(np.abs(g["alpha"][b] - ref["alpha"][0]) <= 1e-6)
        if np.any(np.abs(u - ref["alpha"][0]) < 1e-6):
            print(f"sequence {b}: near-tie decision, skipped")
            continue
        for key in ("accept_len", "path_nodes", "out_tokens"):
            np.testing.assert_array_equal(g[key][b], ref[key][0], err_msg=f"{key} b={b}")
        np.testing.assert_array_equal(g["node_accept"][b].astype(bool), ref["node_accept"][0])


def test_speculative_batch64_small_vocab():
    require_gpu()
    wl = W.WORKLOADS["c5"].scaled(accept_V=4096)
    _spec_case(wl, 6)


def test_speculative_edge_cases():
    require_gpu()
    parents = [-1, 0]
    V = 6
    # 1) P_d(x) = 0 -> alpha = 1 -> accepted for u < 1; fully accepted leaf -> bonus from P_t
    p_t = np.tile(np.array([0.1, 0.2, 0.3, 0.4, 0.0, 0.0], np.float32), (1, 3, 1))
    p_d = np.tile(np.array([0.5, 0.0, 0.0, 0.5, 0.0, 0.0], np.float32), (1, 3, 1))
    toks = np.array([[1, 2]], np.int32)
    # 2) residual all zero -> falls back to P_t (P_t <= P_d everywhere, token rejected)
    p_t2 = np.tile(np.array([0.25, 0.25, 0.0, 0.0, 0.0, 0.0], np.float32), (1, 3, 1))
    p_d2 = np.tile(np.array([0.5, 0.5, 0.0, 0.0, 0.0, 0.0], np.float32), (1, 3, 1))
    toks2 = np.array([[0, 1]], np.int32)
    for pt, pd, tk, u in ((p_t, p_d, toks, [0.999, 0.999, 0.7]),
                          (p_t2, p_d2, toks2, [0.9, 0.0, 0.75]),
                          (p_t2, p_d2, toks2, [0.9, 0.0, 0.0])):
        u = np.array([u], np.float32)
        got = ops.accept_paths(L.MV_ACCEPT_SPECULATIVE, dev_i32(parents), dev_i32(tk), dev(pt), 2,
                               draft=dev(pd), uniforms=dev(u))
        torch.cuda.synchronize()
        ref = O.accept_speculative(pt, pd, tk, parents, u, 2)
        _compare(got, ref, 1, 2, "edge")


def test_speculative_chi_square_on_gpu():
    """First emitted token of a depth-1 chain follows P_target (the rule's purpose)."""
    require_gpu()
    rng = np.random.default_rng(77)
    V, T = 8, 200_000
    pt_row = rng.dirichlet(np.ones(V)).astype(np.float32)
    pd_row = rng.dirichlet(np.ones(V) * 0.7).astype(np.float32)
    p_t = np.broadcast_to(pt_row, (T, 2, V)).copy()
    p_d = np.broadcast_to(pd_row, (T, 2, V)).copy()
    pdn = pd_row.astype(np.float64) / pd_row.astype(np.float64).sum()
    toks = rng.choice(V, size=(T, 1), p=pdn).astype(np.int32)
    u = rng.random((T, 2), dtype=np.float32)
    got = ops.accept_paths(L.MV_ACCEPT_SPECULATIVE, dev_i32([-1]), dev_i32(toks), dev(p_t), 1,
                           draft=dev(p_d), uniforms=dev(u))
    torch.cuda.synchronize()
    first = host(got["out_tokens"])[:, 0]
    ptn = pt_row.astype(np.float64) / pt_row.astype(np.float64).sum()
    assert chisquare(np.bincount(first, minlength=V), ptn * T).pvalue > 1e-3
    sub = slice(0, 2000)
    ref = O.accept_speculative(p_t[sub], p_d[sub], toks[sub], [-1], u[sub], 1)
    np.testing.assert_array_equal(host(got["out_tokens"])[sub], ref["out_tokens"])
