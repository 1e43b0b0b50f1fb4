"""GPU parity of mv_accept_speculative_lm (the speculative rule fed by the target LM head and
the heads' per-depth draft logits, no [B, N+1, V] probabilities) against
oracle.accept_speculative_lm.

Decisions are exact except near a threshold: the GPU takes P_t(x_i) from an fp32 dot product
(bf16 products are exact in fp32; d = 512 terms, relative error well below 1e-5) and the LM
head's fp32 LSE, so a node whose oracle |u - alpha| < 1e-4 and an extra token whose oracle
inverse-CDF position lies within 1e-5 of the total mass from a boundary are counted, and such a
sequence is not compared further.  alpha itself within 1e-4."""
import numpy as np
import pytest
import torch

from oracle import medusa_oracle as O
from medusa_tree_attention_verify_amd import _lib as L
from medusa_tree_attention_verify_amd import ops
from medusa_tree_attention_verify_amd import workloads as W
from tests.gpu_util import dev, dev_i32, host, require_gpu

pytestmark = pytest.mark.gpu

ALPHA_TIE = 1e-4
CDF_TIE = 1e-5


def _ranks(parents):
    seen = {}
    out = []
    for p in parents:
        out.append(seen.get(p, 0))
        seen[p] = seen.get(p, 0) + 1
    return out


def _depths(parents):
    dep = []
    for p in parents:
        dep.append(1 if p < 0 else dep[p] + 1)
    return dep


def _case(B, V, d, widths, seed, noise, draft_bf16=False):
    parents = W.branching_tree(widths)
    N, D = len(parents), len(widths)
    rng = np.random.default_rng(seed)
    x_t = W.normal(seed, "lmspec_x", (B, N + 1, d), 1.0, True)
    w_lm = W.normal(seed, "lmspec_w", (V, d), 3.0 / np.sqrt(d), True)
    z = x_t.astype(np.float64) @ w_lm.astype(np.float64).T          # target logits (input side)
    dep = _depths(parents)
    # draft row of depth k: the target logits of the first row whose children are at depth k+1,
    # plus noise (so that acceptance is neither certain nor impossible)
    rep = [0] + [1 + dep.index(k) for k in range(1, D)]
    draft = np.stack([z[:, rep[k]] for k in range(D)], axis=1) + noise * rng.standard_normal((B, D, V))
    draft = draft.astype(np.float32)
    if draft_bf16:
        draft = W.round_bf16(draft)
    dl64 = draft.astype(np.float64)
    m = dl64.max(axis=-1, keepdims=True)
    draft_lse = (m[..., 0] + np.log(np.exp(dl64 - m).sum(axis=-1))).astype(np.float32)
    # Medusa-style candidates: depth k's tokens are the top widths[k] of the draft row of depth k;
    # a node takes the candidate of its rank among its siblings
    top = np.argsort(-draft, axis=-1, kind="stable")
    rk = _ranks(parents)
    tokens = np.array([[int(top[b, dep[i] - 1, rk[i]]) for i in range(N)] for b in range(B)], np.int32)
    u = rng.random((B, N + 1), dtype=np.float32)
    return parents, D, x_t, w_lm, draft, draft_lse, tokens, u


def _run(B, V, d, widths, seed, noise, draft_bf16=False):
    parents, D, x_t, w_lm, draft, draft_lse, tokens, u = _case(B, V, d, widths, seed, noise, draft_bf16)
    N = len(parents)
    print(f"lmspec B={B} V={V} d={d} N={N} noise={noise} draft_bf16={draft_bf16}", flush=True)
    bf = torch.bfloat16
    xt_d, w_d = dev(x_t, bf), dev(w_lm, bf)
    lse_t = ops.lm_head_argmax(xt_d.reshape(B * (N + 1), d), w_d)["lse"].reshape(B, N + 1)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    got = ops.accept_speculative_lm(dev_i32(parents), dev_i32(tokens), xt_d, w_d, lse_t,
                                    dev(draft, bf if draft_bf16 else torch.float32),
                                    dev(draft_lse), dev(u), D, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    ref = O.accept_speculative_lm(x_t, w_lm, draft, tokens, parents, u, D)
    g = {k: host(v) for k, v in got.items()}
    np.testing.assert_allclose(g["alpha"], ref["alpha"], rtol=0, atol=1e-4)
    # the oracle's terminal rows for the extra token's tie check
    p_t = O._softmax_rows(x_t.astype(np.float64) @ w_lm.astype(np.float64).T)
    dep = _depths(parents)
    ties = 0
    for b in range(B):
        # only nodes whose parent is the prefix or accepted decide anything
        live = np.array([p < 0 or ref["node_accept"][b][p] for p in parents])
        if np.any(live & (np.abs(u[b, :N] - ref["alpha"][b]) < ALPHA_TIE)):
            ties += 1
            continue
        np.testing.assert_array_equal(g["node_accept"][b].astype(bool), ref["node_accept"][b])
        n = int(ref["accept_len"][b])
        assert g["accept_len"][b] == n
        np.testing.assert_array_equal(g["path_nodes"][b], ref["path_nodes"][b])
        np.testing.assert_array_equal(g["out_tokens"][b][:n], ref["out_tokens"][b][:n])
        # extra token: compare unless the oracle's draw sits within CDF_TIE of a boundary
        term = int(ref["path_nodes"][b][n - 1]) if n > 0 else -1
        row = term + 1
        kids = [i for i, p in enumerate(parents) if p == term]
        r = p_t[b, row]
        if kids:
            k = 0 if row == 0 else dep[term]
            dl = draft[b, k].astype(np.float64)
            pd = np.exp(dl - dl.max()) / np.exp(dl - dl.max()).sum()
            res = np.maximum(0.0, r - pd)
            r = res if res.sum() > 0 else r
        c = np.cumsum(r)
        t = float(u[b, N]) * c[-1]
        if np.min(np.abs(c - t)) < CDF_TIE * c[-1]:
            ties += 1
            continue
        assert g["out_tokens"][b][n] == ref["out_tokens"][b][n], f"extra token of sequence {b}"
    print(f"accepted lengths {g['accept_len'].tolist()}, near-ties {ties}")
    assert ties <= max(1, B // 8)
    return g


@pytest.mark.parametrize("B,V,widths,noise", [
    (3, 3001, (4, 3, 2, 1), 0.5),     # odd vocabulary: scalar row passes
    (4, 4096, (4, 3, 2, 1), 0.3),     # float4 row passes
    (2, 1000, (2, 2, 2), 2.0),        # mostly rejected: residuals at shallow rows
    (2, 2048, (3, 1, 1, 1, 1), 0.05), # nearly equal distributions: long accepted paths, leaf draws
])
def test_lmspec_matches_oracle(B, V, widths, noise):
    require_gpu()
    _run(B, V, 512, widths, 80 + B, noise)


def test_lmspec_bf16_draft_logits():
    require_gpu()
    _run(3, 3000, 256, (4, 3, 2, 1), 91, 0.5, draft_bf16=True)


def test_lmspec_llama8b_shape():
    """One sequence at the Llama-3-8B head shape: d = 4096, V = 32000, the 64-node tree."""
    require_gpu()
    _run(1, 32000, 4096, (4, 3, 2, 1), 95, 0.5)


def test_lmspec_bad_token_flags():
    require_gpu()
    parents, D, x_t, w_lm, draft, draft_lse, tokens, u = _case(1, 1000, 256, (2, 2), 97, 0.5)
    tokens[0, 3] = 5000
    bf = torch.bfloat16
    lse_t = ops.lm_head_argmax(dev(x_t, bf).reshape(-1, 256), dev(w_lm, bf))["lse"].reshape(1, -1)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    ops.accept_speculative_lm(dev_i32(parents), dev_i32(tokens), dev(x_t, bf), dev(w_lm, bf), lse_t,
                              dev(draft), dev(draft_lse), dev(u), D, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) & L.MV_DEV_BAD_TOKEN


def _step_check(wl, seed):
    """The whole step with speculative acceptance from the LM head: heads -> tree -> attention ->
    LM head (LSE per verify row) -> speculative acceptance with the heads' logits as the draft ->
    commit.  The step stores the heads' logits in bf16 and takes their LSE from the fp32 logits,
    so the oracle's draft rows are its fp64 head logits rounded to bf16 (its own softmax), and a
    node within 1e-3 of its threshold (or an extra token within 1e-3 of a CDF boundary) is a
    counted near-tie."""
    from medusa_tree_attention_verify_amd.step import VerifyStep
    parents = list(wl.parents)
    N, D = wl.N, wl.D
    bf = torch.bfloat16
    xh, xa, xt = W.gen_heads(wl, seed), W.gen_attention(wl, seed), W.gen_target_head(wl, seed)
    u = W.gen_uniforms(wl, seed)
    heads = O.medusa_heads(xh["h"], xh["w_res"], xh["w_head"], list(wl.head_widths))
    cand = [heads["topk_ids"][:, k, :wl.head_widths[k]] for k in range(wl.K)]
    tree = O.build_tree(parents, cand, list(wl.depth_widths))
    step = VerifyStep(parents=parents, depth_widths=wl.depth_widths, dtype=bf, B=wl.B, Hq=wl.Hq,
                      Hkv=wl.Hkv, dh=wl.dh, max_L=int(xa["prefix_len"].max()),
                      heads={"d": wl.d, "V": wl.V, "K": wl.K, "widths": list(wl.head_widths)},
                      accept="speculative", V=wl.accept_V, target_head=wl.d, commit=True)
    inp = {"h": dev(xh["h"], bf), "w_res": dev(xh["w_res"], bf), "w_head": dev(xh["w_head"], bf),
           "q": dev(xa["q"], bf), "k_cache": dev(xa["k_cache"], bf), "v_cache": dev(xa["v_cache"], bf),
           "prefix_len": dev_i32(xa["prefix_len"]), "x_t": dev(xt["x_t"], bf),
           "w_lm": dev(xt["w_lm"], bf), "uniforms": dev(u)}
    print(f"lmspec step {wl.name} d={wl.d} V={wl.V} seed={seed}", flush=True)
    step.run(inp)
    torch.cuda.synchronize()
    assert int(step.status.item()) == 0
    from tests.gpu_util import check_topk, assert_fp32
    assert check_topk(host(step.cand), heads["logits"], list(wl.head_widths)) == 0
    np.testing.assert_array_equal(host(step.tree["node_tokens"]), tree["tokens"])
    lm = O.lm_head_argmax(xt["x_t"].reshape(-1, wl.d), xt["w_lm"])
    assert_fp32(host(step.target_lse).ravel(), lm["lse"], atol=1e-3, what="target lse")
    draft = W.round_bf16(heads["logits"].astype(np.float32))
    ref = O.accept_speculative_lm(xt["x_t"], xt["w_lm"], draft, tree["tokens"], parents, u, D)
    g = {k: host(v) for k, v in step.acc.items() if v is not None}
    np.testing.assert_allclose(g["alpha"], ref["alpha"], rtol=0, atol=1e-2)
    ties = 0
    for b in range(wl.B):
        # only nodes whose parent is the prefix or accepted decide anything
        live = np.array([p < 0 or ref["node_accept"][b][p] for p in parents])
        if np.any(live & (np.abs(u[b, :N] - ref["alpha"][b]) < 1e-3)):
            ties += 1
            continue
        n = int(ref["accept_len"][b])
        assert g["accept_len"][b] == n
        np.testing.assert_array_equal(g["path_nodes"][b], ref["path_nodes"][b])
        np.testing.assert_array_equal(g["out_tokens"][b][:n], ref["out_tokens"][b][:n])
    if ties == 0:  # the commit of the oracle's accepted paths (a copy: bit-exact)
        k2, v2, p2 = O.kv_commit(xa["k_cache"], xa["v_cache"], xa["prefix_len"],
                                 ref["path_nodes"], ref["accept_len"], N)
        np.testing.assert_array_equal(host(step.prefix_next), p2)
        np.testing.assert_array_equal(host(inp["k_cache"]), k2)
        np.testing.assert_array_equal(host(inp["v_cache"]), v2)
    print("accepted lengths", g["accept_len"].tolist(), "near-ties", ties)
    assert ties <= max(1, wl.B // 4)


def test_step_lmhead_speculative_small():
    require_gpu()
    wl = W.WORKLOADS["c9"].scaled(B=3, d=512, V=3000, accept_V=3000, prefix=(700, 700))
    _step_check(wl, 33)


def test_step_lmhead_speculative_llama8b():
    require_gpu()
    _step_check(W.WORKLOADS["c9"], 9)
