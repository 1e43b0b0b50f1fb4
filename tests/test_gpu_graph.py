"""A whole verify step captured as one HIP graph: every replay equals the eager step.

Replays are interleaved with eager work on the same buffers and with synchronizations, and
each replay's outputs are compared with the eager result (bit-exact: same kernels, same
inputs)."""
import numpy as np
import pytest
import torch

from medusa_tree_attention_verify_amd import workloads as W
from medusa_tree_attention_verify_amd.step import VerifyStep
from tests.gpu_util import assert_bf16, assert_fp32, dev, dev_i32, host, require_gpu

pytestmark = pytest.mark.gpu


def _outputs(step):
    return [t.clone() for t in (step.cand, step.tree["node_tokens"], step.attn_out, step.attn_lse,
                                step.acc["accept_len"], step.acc["out_tokens"])]


@pytest.mark.parametrize("fork,batched", [(False, False), (True, False), (True, True)])
def test_graph_replays_match_eager(fork, batched):
    """fork=True: the attention branch (its own mask build and the attention launch on half of
    the CUs) is a parallel branch of the graph beside the heads and the tree; its replays must
    equal an eager forked step bit for bit (that launch may cut the keys into other chunks than
    the serial one, so its rounding can differ from the serial step's).  batched: 3 sequences with
    64/8 heads and prefixes long enough for the balanced split of the keys."""
    require_gpu()
    if batched:
        wl = W.WORKLOADS["c3"].scaled(B=3, d=512, V=3000, prefix=(700, 3000))
    else:
        wl = W.WORKLOADS["c2"].scaled(d=512, V=3000, prefix=(700, 700))
    dt = torch.bfloat16
    xh = W.gen_heads(wl, 9)
    xa = W.gen_attention(wl, 9)
    target = W.round_bf16(W.gen_target_logits(wl, 9))
    step = VerifyStep(parents=wl.parents, depth_widths=wl.depth_widths, dtype=dt, B=wl.B,
                      Hq=wl.Hq, Hkv=wl.Hkv, dh=wl.dh, max_L=int(xa["prefix_len"].max()),
                      heads={"d": wl.d, "V": wl.V, "K": wl.K, "widths": list(wl.head_widths)},
                      accept="greedy", V=wl.accept_V, commit=fork and not batched)
    inp = {"h": dev(xh["h"], dt), "w_res": dev(xh["w_res"], dt), "w_head": dev(xh["w_head"], dt),
           "q": dev(xa["q"], dt), "k_cache": dev(xa["k_cache"], dt),
           "v_cache": dev(xa["v_cache"], dt), "prefix_len": dev_i32(xa["prefix_len"]),
           "target": dev(target, dt)}
    side = torch.cuda.Stream() if fork else None
    if fork and batched:
        # the forked step against the serial one: the same integer outputs, the attention
        # within the bf16 bar (the two launches may split the keys differently)
        step.run(inp)
        torch.cuda.synchronize()
        serial = _outputs(step)
    step.run(inp, side)
    torch.cuda.synchronize()
    ref = _outputs(step)
    if fork and batched:
        for i in (0, 1, 4, 5):
            assert torch.equal(serial[i], ref[i])
        assert_bf16(host(ref[2]), host(serial[2]), what="forked attention")
        assert_fp32(host(ref[3]), host(serial[3]), atol=1e-3, what="forked attention lse")
    g = step.capture(inp, fork=fork)
    for rep in range(4):
        # eager work in between: clobber the outputs, then replay the graph
        for t in (step.cand, step.tree["node_tokens"], step.acc["accept_len"]):
            t.fill_(-7)
        step.attn_out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(_outputs(step), ref):
            assert torch.equal(a, b), f"replay {rep} differs from the eager step"
        if rep == 1:
            step.run(inp, side)     # an eager step between replays
            torch.cuda.synchronize()
    assert int(step.status.item()) == 0


@pytest.mark.parametrize("draft_input", [False, True])
def test_graph_replays_lmhead_speculative(draft_input):
    """The step with speculative acceptance driven by the target LM head, captured as one graph:
    with the Medusa heads' logits as the draft (3 sequences), or with an input draft whose top
    tokens build the tree (5 sequences: 325 verify rows through the tiled LM head, the one-pass
    top-k with row LSE, the terminal rows of 5 sequences in one pass)."""
    require_gpu()
    if draft_input:
        wl = W.WORKLOADS["c10"].scaled(B=5, d=512, accept_V=3000, prefix=(300, 900))
    else:
        wl = W.WORKLOADS["c9"].scaled(B=3, d=512, V=3000, accept_V=3000, prefix=(700, 700))
    dt = torch.bfloat16
    xa, xt = W.gen_attention(wl, 12), W.gen_target_head(wl, 12)
    inp = {"q": dev(xa["q"], dt), "k_cache": dev(xa["k_cache"], dt), "v_cache": dev(xa["v_cache"], dt),
           "prefix_len": dev_i32(xa["prefix_len"]), "x_t": dev(xt["x_t"], dt),
           "w_lm": dev(xt["w_lm"], dt), "uniforms": dev(W.gen_uniforms(wl, 12))}
    if draft_input:
        inp["draft_logits"] = dev(W.gen_draft_logits(wl, 12), dt)
        heads = None
    else:
        xh = W.gen_heads(wl, 12)
        inp.update(h=dev(xh["h"], dt), w_res=dev(xh["w_res"], dt), w_head=dev(xh["w_head"], dt))
        heads = {"d": wl.d, "V": wl.V, "K": wl.K, "widths": list(wl.head_widths)}
    step = VerifyStep(parents=wl.parents, depth_widths=wl.depth_widths, dtype=dt, B=wl.B,
                      Hq=wl.Hq, Hkv=wl.Hkv, dh=wl.dh, max_L=int(xa["prefix_len"].max()),
                      heads=heads, accept="speculative", V=wl.accept_V, target_head=wl.d)

    def outs():
        return _outputs(step) + [step.acc["alpha"].clone(), step.acc["path_nodes"].clone(),
                                 step.target_lse.clone(), step.head_lse.clone()]
    print(f"graph lmhead speculative draft_input={draft_input}", flush=True)
    step.run(inp)
    torch.cuda.synchronize()
    ref = outs()
    g = step.capture(inp)
    for rep in range(4):
        for t in (step.cand, step.tree["node_tokens"], step.acc["accept_len"], step.acc["out_tokens"]):
            t.fill_(-7)
        step.acc["alpha"].fill_(-1.0)
        step.target_lse.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(outs(), ref):
            assert torch.equal(a, b), f"replay {rep} differs from the eager step"
        if rep == 1:
            step.run(inp)
            torch.cuda.synchronize()
    assert int(step.status.item()) == 0
