"""One whole verify step on the GPU (heads -> tree -> attention -> acceptance -> commit of
the accepted path) vs the oracle."""
import numpy as np
import pytest
import torch

from oracle import medusa_oracle as O
from medusa_tree_attention_verify_amd import workloads as W
from medusa_tree_attention_verify_amd.step import VerifyStep
from tests.gpu_util import assert_bf16, assert_fp32, check_topk, dev, dev_i32, host, require_gpu

pytestmark = pytest.mark.gpu


def _oracle_step(wl, x, target):
    """Oracle of one step; returns candidates, tree, attention, acceptance."""
    parents = list(wl.parents)
    heads = O.medusa_heads(x["h"], x["w_res"], x["w_head"], list(wl.head_widths))
    cand = []
    if wl.lm_width:
        cand.append(np.stack([O.topk_rows(target[b, 0], wl.lm_width)["ids"] for b in range(wl.B)]))
    for k in range(wl.K):
        cand.append(heads["topk_ids"][:, k, :wl.head_widths[k]])
    tree = O.build_tree(parents, cand, list(wl.depth_widths))
    return heads, cand, tree


def _check_step(wl, seed, attn_select=None, fork=False):
    """One GPU step vs the oracle.  ``attn_select`` = (b, h, i) rows whose attention output
    is compared (all rows when None); everything else is compared in full.  ``fork`` runs the
    step forked (the attention branch, with the launch on half of the CUs, on a second stream)."""
    parents = list(wl.parents)
    dt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    xh = W.gen_heads(wl, seed)
    xa = W.gen_attention(wl, seed)
    if wl.target_head:
        xt = W.gen_target_head(wl, seed)
        heads, cand, tree = _oracle_step(wl, xh, None)
        x_t = xt["x_t"].copy()
        if wl.plant_p > 0:
            x_t = W.plant_target_head(x_t, xt["w_lm"], parents, tree["tokens"], seed, wl.plant_p)
        lm = O.lm_head_argmax(x_t.reshape(-1, wl.d), xt["w_lm"])
        target = lm["logits"].reshape(wl.B, wl.N + 1, wl.accept_V)
    else:
        target = W.gen_target_logits(wl, seed)
        heads, cand, tree = _oracle_step(wl, xh, target)
        if wl.plant_p > 0:
            target = W.plant_greedy(target, parents, tree["tokens"], seed, wl.plant_p)
        if wl.dtype == "bf16":
            target = W.round_bf16(target)
    step = VerifyStep(parents=parents, depth_widths=wl.depth_widths, dtype=dt, B=wl.B, Hq=wl.Hq,
                      Hkv=wl.Hkv, dh=wl.dh, max_L=int(xa["prefix_len"].max()),
                      heads={"d": wl.d, "V": wl.V, "K": wl.K, "widths": list(wl.head_widths)},
                      lm_width=wl.lm_width, accept="greedy", V=wl.accept_V,
                      target_head=wl.d if wl.target_head else None, commit=True)
    inp = {"h": dev(xh["h"], dt), "w_res": dev(xh["w_res"], dt), "w_head": dev(xh["w_head"], dt),
           "q": dev(xa["q"], dt), "k_cache": dev(xa["k_cache"], dt),
           "v_cache": dev(xa["v_cache"], dt), "prefix_len": dev_i32(xa["prefix_len"])}
    if wl.target_head:
        inp.update(x_t=dev(x_t.reshape(wl.B, wl.N + 1, wl.d), torch.bfloat16),
                   w_lm=dev(xt["w_lm"], torch.bfloat16))
        # the greedy tokens must not hinge on a near-tie between the two largest logits
        srt = np.sort(target, axis=-1)
        assert np.all(srt[..., -1] - srt[..., -2] > 1e-4 * np.maximum(1.0, np.abs(srt[..., -1])))
    else:
        inp["target"] = dev(target, dt)
    print(f"step {wl.name} seed={seed} fork={fork}", flush=True)
    step.run(inp, torch.cuda.Stream() if fork else None)
    torch.cuda.synchronize()
    assert int(step.status.item()) == 0
    # heads: ids exact (near-ties counted), candidate tokens and tree exact
    off = 1 if wl.lm_width else 0
    ties = check_topk(host(step.cand)[:, off:, :], heads["logits"],
                      [w for w in wl.head_widths])
    assert ties == 0, "a near-tie changes the tree; the step comparison below would not hold"
    np.testing.assert_array_equal(host(step.tree["node_tokens"]), tree["tokens"])
    np.testing.assert_array_equal(host(step.tree["depth"]), tree["depth"])
    ref_att = O.tree_attention(xa["q"], xa["k_cache"], xa["v_cache"], xa["prefix_len"], tree["anc"],
                               select=attn_select)
    got_o, got_l = host(step.attn_out), host(step.attn_lse)
    ref_o, ref_l = ref_att["out"], ref_att["lse"]
    if attn_select is not None:
        bb, hh, ii = np.array(attn_select).T
        got_o, ref_o = got_o[bb, ii, hh], ref_o[bb, ii, hh]
        got_l, ref_l = got_l[bb, hh, ii], ref_l[bb, hh, ii]
    if wl.dtype == "f32":
        assert_fp32(got_o, ref_o, what="attention")
    else:
        assert_bf16(got_o, ref_o, what="attention")
    assert_fp32(got_l, ref_l, atol=1e-4 if wl.dtype == "f32" else 1e-3, what="lse")
    ref_acc = O.accept_greedy(target, tree["tokens"], parents, wl.D)
    for k in ("accept_len", "path_nodes", "out_tokens"):
        np.testing.assert_array_equal(host(step.acc[k]), ref_acc[k], err_msg=k)
    # the step ends with the commit of the accepted path (a copy: bit-exact)
    k2, v2, p2 = O.kv_commit(xa["k_cache"], xa["v_cache"], xa["prefix_len"],
                             ref_acc["path_nodes"], ref_acc["accept_len"], wl.N)
    np.testing.assert_array_equal(host(step.prefix_next), p2)
    np.testing.assert_array_equal(host(inp["prefix_len"]), xa["prefix_len"])
    np.testing.assert_array_equal(host(inp["k_cache"]), k2)
    np.testing.assert_array_equal(host(inp["v_cache"]), v2)
    return host(step.acc["accept_len"])


def test_step_tiny_fp32():
    require_gpu()
    _check_step(W.WORKLOADS["c1"], 1)


@pytest.mark.parametrize("fork", [False, True], ids=["serial", "forked"])
def test_step_llama8b_full(fork):
    require_gpu()
    lens = _check_step(W.WORKLOADS["c2"], 2, fork=fork)
    print("accepted length", lens.tolist())


def test_step_target_head_small():
    """A whole step whose greedy target comes from the LM head over the verify rows."""
    require_gpu()
    wl = W.WORKLOADS["c6"].scaled(d=512, V=3000, accept_V=3000, prefix=(700, 700))
    lens = _check_step(wl, 31)
    print("accept lengths", lens.tolist())


def test_step_target_head_llama8b_full():
    """The Llama-3-8B-shaped step with the target LM head (W_lm 32000 x 4096)."""
    require_gpu()
    lens = _check_step(W.WORKLOADS["c6"], 6)
    print("accept lengths", lens.tolist())


@pytest.mark.parametrize("fork", [False, True], ids=["serial", "forked"])
def test_step_70b_share_full(fork):
    """The 70B-shaped one-GPU share at full size (batch 8, 64/8 heads, prefixes in
    [8192, 32768], d = 8192, 4 heads over V = 32000): all 32 (sequence, head) candidate lists,
    the tree tokens, the accepted lengths, paths and tokens of all 8 sequences and the
    committed caches exactly; the attention on sampled rows of every sequence (the oracle
    computes each row from the whole prefix, one (sequence, KV head) slice at a time)."""
    require_gpu()
    wl = W.WORKLOADS["c3"]
    rng = np.random.default_rng(33)
    sel = []
    for b in range(wl.B):
        sel += [(b, int(rng.integers(wl.Hq)), int(rng.integers(wl.N))) for _ in range(3)]
        sel += [(b, int(rng.integers(wl.Hq)), wl.N - 1)]
    lens = _check_step(wl, 3, attn_select=sel, fork=fork)
    print("accepted lengths", lens.tolist())
