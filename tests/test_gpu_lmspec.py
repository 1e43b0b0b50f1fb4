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
    (20, 1000, (4, 3, 2, 1), 0.5),    # terminal rows over two 16-row column tiles
    (130, 777, (2, 2), 1.0),          # ... and over two groups of 128 rows
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


def _step_check(wl, seed, seqs=None):
    """The whole step with speculative acceptance from the LM head: candidates -> tree ->
    attention -> LM head (LSE per verify row) -> speculative acceptance -> commit.

    With Medusa heads the draft of depth k is head k's logits: the step stores them in bf16 and
    takes their LSE from the fp32 logits, so the oracle's draft rows are its fp64 head logits
    rounded to bf16 (its own softmax).  Without heads the draft is an input [B, D, V] of bf16
    logits, which both sides read as given, and the candidates are its rows' top tokens.  A
    node within 1e-3 of its threshold is a counted near-tie.  ``seqs`` restricts the oracle to
    those sequences (every sequence is independent of the others)."""
    from medusa_tree_attention_verify_amd.step import VerifyStep
    from tests.gpu_util import check_topk, assert_fp32
    parents = list(wl.parents)
    N, D = wl.N, wl.D
    bf = torch.bfloat16
    seqs = list(range(wl.B)) if seqs is None else list(seqs)
    xa, xt = W.gen_attention(wl, seed), W.gen_target_head(wl, seed)
    u = W.gen_uniforms(wl, seed)
    inp = {"q": dev(xa["q"], bf), "k_cache": dev(xa["k_cache"], bf), "v_cache": dev(xa["v_cache"], bf),
           "prefix_len": dev_i32(xa["prefix_len"]), "x_t": dev(xt["x_t"], bf),
           "w_lm": dev(xt["w_lm"], bf), "uniforms": dev(u)}
    if wl.has_heads:
        xh = W.gen_heads(wl, seed)
        heads = O.medusa_heads(xh["h"][seqs], xh["w_res"], xh["w_head"], list(wl.head_widths))
        cand = [heads["topk_ids"][:, k, :wl.head_widths[k]] for k in range(wl.K)]
        draft = W.round_bf16(heads["logits"].astype(np.float32))
        inp.update(h=dev(xh["h"], bf), w_res=dev(xh["w_res"], bf), w_head=dev(xh["w_head"], bf))
        hd = {"d": wl.d, "V": wl.V, "K": wl.K, "widths": list(wl.head_widths)}
    else:
        dl = W.gen_draft_logits(wl, seed)
        draft = dl[seqs]
        cand = [np.stack([O.topk_rows(draft[i, k], wl.depth_widths[k])["ids"]
                          for i in range(len(seqs))]) for k in range(D)]
        inp["draft_logits"] = dev(dl, bf)
        hd = None
    tree = O.build_tree(parents, cand, list(wl.depth_widths))
    step = VerifyStep(parents=parents, depth_widths=wl.depth_widths, dtype=bf, B=wl.B, Hq=wl.Hq,
                      Hkv=wl.Hkv, dh=wl.dh, max_L=int(xa["prefix_len"].max()), heads=hd,
                      accept="speculative", V=wl.accept_V, target_head=wl.d, commit=True)
    print(f"lmspec step {wl.name} B={wl.B} d={wl.d} V={wl.accept_V} seed={seed} "
          f"sequences {len(seqs)}", flush=True)
    step.run(inp)
    torch.cuda.synchronize()
    assert int(step.status.item()) == 0
    if wl.has_heads:
        assert check_topk(host(step.cand)[seqs], heads["logits"], list(wl.head_widths)) == 0
    else:   # top tokens of the given bf16 rows: exact on both sides
        for k in range(D):
            np.testing.assert_array_equal(host(step.cand)[seqs, k, :wl.depth_widths[k]], cand[k])
    np.testing.assert_array_equal(host(step.tree["node_tokens"])[seqs], tree["tokens"])
    x_t = xt["x_t"][seqs]
    lm = O.lm_head_argmax(x_t.reshape(-1, wl.d), xt["w_lm"])
    assert_fp32(host(step.target_lse)[seqs].ravel(), lm["lse"], atol=1e-3, what="target lse")
    ref = O.accept_speculative_lm(x_t, xt["w_lm"], draft, tree["tokens"], parents, u[seqs], D)
    g = {k: host(v)[seqs] for k, v in step.acc.items() if v is not None}
    np.testing.assert_allclose(g["alpha"], ref["alpha"], rtol=0, atol=1e-2)
    ties = 0
    for i, b in enumerate(seqs):
        # only nodes whose parent is the prefix or accepted decide anything
        live = np.array([p < 0 or ref["node_accept"][i][p] for p in parents])
        if np.any(live & (np.abs(u[b, :N] - ref["alpha"][i]) < 1e-3)):
            ties += 1
            continue
        n = int(ref["accept_len"][i])
        assert g["accept_len"][i] == n
        np.testing.assert_array_equal(g["path_nodes"][i], ref["path_nodes"][i])
        np.testing.assert_array_equal(g["out_tokens"][i][:n], ref["out_tokens"][i][:n])
        # the extra token: the inverse CDF of the residual (or target) row at u[b, N], the same
        # up to a draw that lands within rounding of a CDF step (counted with the near-ties)
        if g["out_tokens"][i][n] != ref["out_tokens"][i][n]:
            ties += 1
    if ties == 0:  # the commit of the oracle's accepted paths (a copy: bit-exact)
        k2, v2, p2 = O.kv_commit(xa["k_cache"][seqs], xa["v_cache"][seqs], xa["prefix_len"][seqs],
                                 ref["path_nodes"], ref["accept_len"], N)
        np.testing.assert_array_equal(host(step.prefix_next)[seqs], p2)
        np.testing.assert_array_equal(host(inp["k_cache"])[seqs], k2)
        np.testing.assert_array_equal(host(inp["v_cache"])[seqs], v2)
    print("accepted lengths", g["accept_len"].tolist(), "near-ties", ties)
    assert ties <= max(1, len(seqs) // 4)


def test_step_lmhead_speculative_small():
    require_gpu()
    wl = W.WORKLOADS["c9"].scaled(B=3, d=512, V=3000, accept_V=3000, prefix=(700, 700))
    _step_check(wl, 33)


def test_step_lmhead_speculative_llama8b():
    require_gpu()
    _step_check(W.WORKLOADS["c9"], 9)


def test_step_lmhead_speculative_draft_input_small():
    """The batched serving step driven by the LM head, scaled down: 5 sequences (325 verify
    rows, so the LM head runs its tiled kernel), d = 512, V = 3000, ragged prefixes; the draft
    is an input of per-depth logits."""
    require_gpu()
    wl = W.WORKLOADS["c10"].scaled(B=5, d=512, accept_V=3000, prefix=(300, 900))
    _step_check(wl, 41)


def test_step_lmhead_speculative_serving_b64_sampled():
    """The full serving step driven by the LM head (64 sequences, W_lm 128256 x 4096, 4160
    verify rows through the tiled kernel with 256-row target tiles): the GPU runs every
    sequence, the oracle recomputes 8 of them."""
    require_gpu()
    wl = W.WORKLOADS["c10"]
    _step_check(wl, 10, seqs=[0, 9, 17, 31, 40, 52, 60, 63])
