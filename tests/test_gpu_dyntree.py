"""GPU parity of the dynamic (confidence-ranked) tree (mv_build_dynamic_tree) against the
oracle, and of attention and acceptance on per-sequence trees."""
import math

import numpy as np
import pytest
import torch

from oracle import medusa_oracle as O
from medusa_tree_attention_verify_amd import _lib as L
from medusa_tree_attention_verify_amd import ops
from medusa_tree_attention_verify_amd import workloads as W
from tests.gpu_util import assert_fp32, dev, dev_i32, host, require_gpu

pytestmark = pytest.mark.gpu


def _heads(B, D, s_max, V, seed, std=2.0):
    """Candidates of D heads: the top s_max tokens of N(0, std) logits, with each head's LSE."""
    logits = W.normal(seed, "dyn_logits", (B, D, V), std)
    ids = np.argsort(-logits, axis=2, kind="stable")[:, :, :s_max].astype(np.int32)
    vals = np.take_along_axis(logits, ids, axis=2).astype(np.float32)
    lse = np.log(np.exp(logits.astype(np.float64)).sum(axis=2)).astype(np.float32)
    return ids, vals, lse


def _mask_bits(anc, N):
    W_ = (N + 31) // 32
    m = np.zeros((N, W_), dtype=np.uint32)
    for i, a in enumerate(anc):
        for j in a:
            m[i, j // 32] |= np.uint32(1 << (j % 32))
    return m


def _check(got, ref, N):
    B = len(ref["parents"])
    g = {k: host(v) for k, v in got.items()}
    for b in range(B):
        np.testing.assert_array_equal(g["parents"][b], ref["parents"][b], err_msg=f"parents b={b}")
        np.testing.assert_array_equal(g["depth"][b], ref["depth"][b])
        np.testing.assert_array_equal(g["node_tokens"][b], ref["tokens"][b])
        np.testing.assert_array_equal(g["anc_mask"][b].view(np.uint32), _mask_bits(ref["anc"][b], N))
        np.testing.assert_array_equal(g["node_logp"][b],
                                      np.array(ref["score"][b], np.float64).astype(np.float32))


@pytest.mark.parametrize("B,D,s,N,V", [
    (4, 4, (10, 10, 10, 10), 64, 1000),
    (2, 3, (6, 5, 3), 17, 500),
    (3, 4, (16, 16, 16, 16), 256, 4000),
    (2, 15, (2,) * 15, 256, 300),        # deepest trees, the largest node count
    (1, 1, (16,), 16, 100),              # every path
    (5, 6, (4, 3, 3, 2, 2, 2), 40, 700),
    (2, 15, (2,) * 15, 64, 300),         # the sorted-frontier selection (N <= 64), deepest keys
    (3, 4, (16, 16, 16, 16), 65, 4000),  # the smallest N of the LDS-frontier selection
])
def test_dynamic_tree_matches_oracle(B, D, s, N, V):
    require_gpu()
    s_max = max(s)
    print(f"dynamic tree B={B} D={D} s={s} N={N}", flush=True)
    ids, vals, lse = _heads(B, D, s_max, V, B * 100 + N)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    got = ops.build_dynamic_tree(dev_i32(ids), dev(vals), dev(lse), N, s_per_depth=s,
                                 status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    _check(got, O.dynamic_tree(ids, vals, lse, s, N), N)
    print("depth histogram", np.bincount(host(got["depth"]).ravel()).tolist())


def test_dynamic_tree_exact_ties():
    """Powers-of-two probabilities: joint scores tie exactly, so depth and then ranks decide
    (the oracle's hand example)."""
    require_gpu()
    ln2 = np.float32(math.log(2.0))
    k = np.array([[[1, 2, 3], [1, 2, 2], [1, 1, 9]]], np.float32)
    vals = -k * ln2
    ids = np.array([[[10, 11, 12], [20, 21, 22], [30, 31, 32]]], np.int32)
    for N, want in ((4, [-1, -1, -1, 0]), (6, [-1, -1, -1, 0, 0, 0]),
                    (8, [-1, -1, -1, 0, 0, 0, 1, 3])):
        got = ops.build_dynamic_tree(dev_i32(ids), dev(vals), None, N, s_per_depth=(3, 3, 2))
        torch.cuda.synchronize()
        assert host(got["parents"])[0].tolist() == want
        _check(got, O.dynamic_tree(ids, vals, None, (3, 3, 2), N), N)


def test_per_sequence_trees_attention_and_acceptance():
    """Each sequence verifies its own dynamic tree: attention with per-sequence masks (fp32)
    and greedy acceptance with per-sequence parent arrays, against the oracle run sequence by
    sequence on its own tree."""
    require_gpu()
    B, D, s, N, V = 3, 4, (6, 4, 3, 2), 24, 800
    ids, vals, lse = _heads(B, D, max(s), V, 5)
    tree = ops.build_dynamic_tree(dev_i32(ids), dev(vals), dev(lse), N, s_per_depth=s)
    ref_tree = O.dynamic_tree(ids, vals, lse, s, N)
    wl = W.Workload(name="dyn-attn", dtype="f32", B=B, Hq=8, Hkv=2, dh=64,
                    parents=tuple(range(-1, N - 1)), prefix=(30, 400), depth_widths=s)
    x = W.gen_attention(wl, 6)
    out, lse_a = ops.tree_attn_verify(dev(x["q"]), dev(x["k_cache"]), dev(x["v_cache"]),
                                      dev_i32(x["prefix_len"]), tree["anc_mask"],
                                      int(x["prefix_len"].max()))
    # greedy targets planted against each sequence's own tree
    target = W.normal(7, "dyn_target", (B, N + 1, V), 2.0)
    toks = np.array(ref_tree["tokens"], np.int32)
    for b in range(B):
        target[b:b + 1] = W.plant_greedy(target[b:b + 1], ref_tree["parents"][b], toks[b:b + 1],
                                         8 + b, 0.7)
    acc = ops.accept_paths(L.MV_ACCEPT_GREEDY, tree["parents"], tree["node_tokens"], dev(target), D)
    torch.cuda.synchronize()
    _check(tree, ref_tree, N)
    o, l = host(out), host(lse_a)
    for b in range(B):
        sl = slice(b, b + 1)
        ra = O.tree_attention(x["q"][sl], x["k_cache"][sl], x["v_cache"][sl], x["prefix_len"][sl],
                              ref_tree["anc"][b])
        assert_fp32(o[b], ra["out"][0], what=f"attention b={b}")
        assert_fp32(l[b], ra["lse"][0], what=f"lse b={b}")
        rg = O.accept_greedy(target[sl], toks[sl], ref_tree["parents"][b], D)
        for key in ("accept_len", "path_nodes", "out_tokens"):
            np.testing.assert_array_equal(host(acc[key])[b], rg[key][0], err_msg=f"{key} b={b}")
    print("accept lengths", host(acc["accept_len"]).tolist())


def _boundary_gap(logits, widths, N):
    """fp64 joint log-probability of the N-th most probable candidate path minus that of the
    (N+1)-th (every path of ranks r_k < widths[k]; log-probabilities from the heads' own
    logits, clamped at 0)."""
    logp = []
    for k, z in enumerate(logits):
        m = z.max()
        lse = m + np.log(np.exp(z - m).sum())
        logp.append(np.minimum(0.0, np.sort(z)[::-1][:widths[k]] - lse))
    scores, level = [], np.zeros(1)
    for k in range(len(widths)):
        level = (level[:, None] + logp[k][None, :]).ravel()
        scores.append(level)
    s = np.sort(np.concatenate(scores))[::-1]
    return float(s[N - 1] - s[N]) if len(s) > N else float("inf")


@pytest.mark.parametrize("name,scale", [("c8", dict(d=512, V=3000, accept_V=3000, prefix=(700, 700))),
                                        ("c8", None)])
def test_step_with_dynamic_tree(name, scale):
    """The whole step in dynamic-tree mode (heads -> per-sequence tree -> attention ->
    greedy acceptance -> commit) against the oracle; the full size is the Llama-3-8B-shaped
    step with 10 candidates per head and 64 nodes."""
    require_gpu()
    from medusa_tree_attention_verify_amd.step import VerifyStep
    from tests.gpu_util import assert_bf16, check_topk
    wl = W.WORKLOADS[name] if scale is None else W.WORKLOADS[name].scaled(**scale)
    N, D = wl.dynamic_nodes, wl.D
    seed = 41
    print(f"dynamic step d={wl.d} V={wl.V} N={N}", flush=True)
    xh = W.gen_heads(wl, seed)
    xa = W.gen_attention(wl, seed)
    heads = O.medusa_heads(xh["h"], xh["w_res"], xh["w_head"], list(wl.head_widths))
    dyn = O.dynamic_tree(heads["topk_ids"], heads["topk_vals"], heads["lse"],
                         list(wl.head_widths), N)
    target = W.gen_target_logits(wl, seed)
    for b in range(wl.B):
        target[b:b + 1] = W.plant_greedy(target[b:b + 1], dyn["parents"][b],
                                         np.array([dyn["tokens"][b]]), seed + b, wl.plant_p)
    target = W.round_bf16(target)
    step = VerifyStep(parents=None, depth_widths=wl.depth_widths, dtype=torch.bfloat16, B=wl.B,
                      Hq=wl.Hq, Hkv=wl.Hkv, dh=wl.dh, max_L=int(xa["prefix_len"].max()),
                      heads={"d": wl.d, "V": wl.V, "K": wl.K, "widths": list(wl.head_widths)},
                      accept="greedy", V=wl.accept_V, commit=True, dynamic_nodes=N)
    bf = torch.bfloat16
    inp = {"h": dev(xh["h"], bf), "w_res": dev(xh["w_res"], bf), "w_head": dev(xh["w_head"], bf),
           "q": dev(xa["q"], bf), "k_cache": dev(xa["k_cache"], bf),
           "v_cache": dev(xa["v_cache"], bf), "prefix_len": dev_i32(xa["prefix_len"]),
           "target": dev(target, bf)}
    step.run(inp)
    torch.cuda.synchronize()
    assert int(step.status.item()) == 0
    assert check_topk(host(step.cand), heads["logits"], list(wl.head_widths)) == 0, \
        "a near-tie changes the candidates; the comparison below would not hold"
    # the tree is built from the GPU's fp32 candidate logits and LSE: the oracle builds it from
    # those same values (exact parity), and it is also compared with the fp64 heads' tree
    ref = O.dynamic_tree(host(step.cand), host(step.cand_vals), host(step.head_lse),
                         list(wl.head_widths), N)
    # ... and equal to the tree of the fp64 heads whenever no two candidate paths are so close
    # in fp64 score that fp32 logits could reorder them at the N-th place
    for b in range(wl.B):
        gap = _boundary_gap(heads["logits"][b], list(wl.head_widths), N)
        print(f"b={b}: score gap at the N-th path {gap:.3g}")
        if gap > 1e-3:
            assert ref["parents"][b] == dyn["parents"][b], f"b={b}: tree shape"
            assert ref["tokens"][b] == dyn["tokens"][b], f"b={b}: tree tokens"
    for b in range(wl.B):
        sl = slice(b, b + 1)
        np.testing.assert_array_equal(host(step.parents)[b], ref["parents"][b])
        np.testing.assert_array_equal(host(step.tree["node_tokens"])[b], ref["tokens"][b])
        toks = np.array([ref["tokens"][b]])
        ra = O.tree_attention(xa["q"][sl], xa["k_cache"][sl], xa["v_cache"][sl],
                              xa["prefix_len"][sl], ref["anc"][b])
        assert_bf16(host(step.attn_out)[b], ra["out"][0], what=f"attention b={b}")
        rg = O.accept_greedy(target[sl], toks, ref["parents"][b], D)
        for key in ("accept_len", "path_nodes", "out_tokens"):
            np.testing.assert_array_equal(host(step.acc[key])[b], rg[key][0], err_msg=key)
        k2, v2, p2 = O.kv_commit(xa["k_cache"][sl], xa["v_cache"][sl], xa["prefix_len"][sl],
                                 rg["path_nodes"], rg["accept_len"], N)
        np.testing.assert_array_equal(host(step.prefix_next)[b], p2[0])
        np.testing.assert_array_equal(host(inp["k_cache"])[b], k2[0])
    print("accept lengths", host(step.acc["accept_len"]).tolist(),
          "depths", np.bincount(host(step.tree["depth"]).ravel()).tolist())
