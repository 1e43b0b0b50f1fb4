"""One Medusa tree-verification step on the GPU: heads -> tree -> attention -> acceptance
(-> commit of the accepted path into the KV cache, with ``commit=True``).

All buffers (outputs and workspaces) are allocated once in ``VerifyStep.__init__``.
``bind(inp)`` turns one set of device inputs into one pre-marshalled C-ABI call per part
(heads residual, heads projection, heads selection, tree, attention, target LM head,
acceptance, commit; those the step has), so a step costs a few ctypes calls and no Python-side
checks or allocation.  The candidate tokens of depth k come from Medusa head k; with ``lm_width > 0`` the depth-1 candidates are instead the top ``lm_width`` tokens
of the target's first row (the base model's own head, which predicts the next token) and
the Medusa heads supply depths 2..D.

With ``commit=True`` the step ends by moving the accepted path's K/V rows to the front of the
tree block (in the caller's ``k_cache`` / ``v_cache``) and writing the grown prefix lengths to
``prefix_next``; ``prefix_len`` itself is left alone, so a replayed step sees the same prefix.
"""
from __future__ import annotations

from typing import Callable, Dict, List, Optional, Sequence

import torch

from . import _lib as L
from . import ops


def _p(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


class VerifyStep:
    PARTS = ("heads_residual", "heads_projection", "heads_select", "tree", "attn_mask",
             "attention", "target_head", "accept", "commit")
    # the attention branch of a forked step: it needs only the tree's static ancestor mask,
    # not the heads' candidates, so it can run beside the heads on a second stream
    BRANCH = ("attn_mask", "attention")

    def __init__(self, *, parents: Optional[Sequence[int]], depth_widths: Sequence[int],
                 dtype: torch.dtype, B: int, Hq: int, Hkv: int, dh: int, max_L: int,
                 heads: Optional[Dict[str, object]] = None, lm_width: int = 0,
                 accept: str = "greedy", V: int = 0, tokens_given: bool = False,
                 target_head: Optional[int] = None, commit: bool = False,
                 dynamic_nodes: Optional[int] = None, device="cuda"):
        # dynamic_nodes = N: each sequence's tree is its N most probable head-candidate paths
        # (built every step from the heads' candidates); parents is then unused
        self.dynamic = dynamic_nodes
        if dynamic_nodes:
            if heads is None or lm_width or tokens_given or heads["K"] != len(depth_widths):
                raise ValueError("a dynamic tree is built from the Medusa heads' candidates "
                                 "(one head per depth)")
            self.parents_list = None
            self.N = int(dynamic_nodes)
        else:
            ops.validate_parents(parents)
            self.parents_list = [int(p) for p in parents]
            self.N = len(parents)
        self.D = len(depth_widths)
        self.depth_widths = [int(s) for s in depth_widths]
        self.s_max = max(self.depth_widths)
        self.B, self.Hq, self.Hkv, self.dh, self.max_L = B, Hq, Hkv, dh, max_L
        self.dtype = dtype
        self.dt = L.MV_BF16 if dtype == torch.bfloat16 else L.MV_F32
        self.accept = accept
        self.mode = {"speculative": L.MV_ACCEPT_SPECULATIVE,
                     "multicand": L.MV_ACCEPT_MULTICAND}.get(accept, L.MV_ACCEPT_GREEDY)
        self.V = V
        self.lm_width = lm_width
        self.heads = heads  # {"d":, "V":, "K":, "widths":}
        self.tokens_given = tokens_given  # node tokens come with the inputs (no heads)
        # target from the LM head (hidden width target_head): inputs x_t [B, N+1, d] and
        # w_lm [V, d].  Greedy: its argmax ids feed greedy acceptance.  Speculative: its LSE per
        # row and the draft logits of each depth feed the speculative rule; the draft rows are
        # the heads' own logits, or without heads an input draft_logits [B, D, V] (a separate
        # draft's per-depth logits), whose top candidates then build the tree.  No
        # [B, N+1, V] tensor is made either way
        self.target_head = target_head
        self.draft_input = bool(target_head) and accept == "speculative" and heads is None
        dev = torch.device(device)
        self.device = dev
        if self.dynamic:
            self.parents = torch.empty((B, self.N), dtype=torch.int32, device=dev)
        else:
            self.parents = torch.tensor(self.parents_list, dtype=torch.int32, device=dev)
        self.status = torch.zeros(1, dtype=torch.int32, device=dev)
        N, W = self.N, (self.N + 31) // 32
        self.cand = torch.full((B, self.D, self.s_max), -1, dtype=torch.int32, device=dev)
        self.cand_vals = torch.empty((B, self.D, self.s_max), dtype=torch.float32, device=dev)
        if self.dynamic:
            self.tree = {"anc_mask": torch.empty((B, N, W), dtype=torch.int32, device=dev),
                         "depth": torch.empty((B, N), dtype=torch.int32, device=dev),
                         "node_tokens": torch.empty((B, N), dtype=torch.int32, device=dev),
                         "node_logp": torch.empty((B, N), dtype=torch.float32, device=dev)}
        else:
            self.tree = {"anc_mask": torch.empty((N, W), dtype=torch.int32, device=dev),
                         "depth": torch.empty(N, dtype=torch.int32, device=dev),
                         "node_tokens": torch.empty((B, N), dtype=torch.int32, device=dev)}
        # a second ancestor mask, written by the attention branch of a forked step (the main
        # branch's tree call writes its own copy together with the tokens)
        self.attn_anc = (torch.empty((N, W), dtype=torch.int32, device=dev)
                         if not self.dynamic else None)
        self.attn_out = torch.empty((B, N, Hq, dh), dtype=dtype, device=dev)
        self.attn_lse = torch.empty((B, Hq, N), dtype=torch.float32, device=dev)
        self.ws_heads = ops.Workspace(dev)
        self.ws_attn = ops.Workspace(dev)
        self.ws_accept = ops.Workspace(dev)
        if heads is not None:
            d, Vh, K = heads["d"], heads["V"], heads["K"]
            self.head_lse = torch.empty((B, K), dtype=torch.float32, device=dev)
            self.ws_heads.get(ops.heads_workspace_bytes(self.dt, B, d, Vh, K, self.s_max))
            self._s_heads = L.int_array(heads["widths"])
        self.ws_attn.get(ops.attn_workspace_bytes(self.dt, B, N, Hq, Hkv, dh, max_L))
        if self.can_fork():  # a forked step runs the attention launch on half of the CUs
            self.ws_attn.get(ops.attn_workspace_bytes(self.dt, B, N, Hq, Hkv, dh, max_L, True))
        self._s_depth = L.int_array(self.depth_widths)
        if target_head:
            if accept not in ("greedy", "speculative") or dtype != torch.bfloat16:
                raise ValueError("the target LM head feeds bf16 greedy or speculative acceptance")
            if accept == "speculative" and (lm_width or dynamic_nodes or tokens_given or
                                            (heads is not None and heads["K"] != self.D)):
                raise ValueError("speculative acceptance from the LM head takes its draft and "
                                 "candidates from per-depth logits: the Medusa heads (one head "
                                 "per depth) or an input draft_logits [B, D, V]")
            self.ws_lm = ops.Workspace(dev)
            self.ws_lm.get(ops.lm_head_workspace_bytes(B * (N + 1), target_head, V))
            self.target_ids = torch.empty((B, N + 1), dtype=torch.int32, device=dev)
            self.target_lse = torch.empty((B, N + 1), dtype=torch.float32, device=dev)
            if accept == "speculative" and heads is not None:
                # the heads' logits: draft row of depth k = head k
                self.draft_logits = torch.empty((B, heads["K"], heads["V"]), dtype=dtype,
                                                device=dev)
            elif accept == "speculative":  # LSE of each input draft row
                self.head_lse = torch.empty((B, self.D), dtype=torch.float32, device=dev)
        if commit and accept == "none":
            raise ValueError("the commit needs an acceptance rule")
        self.commit = commit
        self.prefix_next = torch.empty(B, dtype=torch.int32, device=dev) if commit else None
        self.spec_lm = bool(target_head) and accept == "speculative"
        if self.spec_lm:
            self.ws_accept.get(L.lib().mv_accept_speculative_lm_workspace(B, N, V))
        elif accept != "none":
            self.ws_accept.get(ops.accept_workspace_bytes(self.mode, B, N, V))
        if accept != "none":
            self.acc = {"accept_len": torch.empty(B, dtype=torch.int32, device=dev),
                        "path_nodes": torch.empty((B, self.D), dtype=torch.int32, device=dev),
                        "out_tokens": torch.empty((B, self.D + 1), dtype=torch.int32, device=dev),
                        "node_accept": torch.empty((B, N), dtype=torch.uint8, device=dev),
                        "alpha": torch.empty((B, N), dtype=torch.float32, device=dev)
                        if self.mode != L.MV_ACCEPT_GREEDY else None}

    @staticmethod
    def _ws(w: ops.Workspace):
        return (None, 0) if w.buf is None else (w.buf.data_ptr(), w.buf.numel())

    def can_fork(self) -> bool:
        return not self.dynamic

    def bind(self, inp: Dict[str, torch.Tensor], branch_stream=None) -> Dict[str, Callable[[], None]]:
        """Pre-marshalled calls of one step on ``inp`` (device tensors: h, w_res, w_head when
        the step has heads; q, k_cache, v_cache, prefix_len; target (+ draft, uniforms);
        node_tokens when the tokens are given; x_t, w_lm with the target LM head, and
        draft_logits [B, D, V] for its speculative rule without heads).  Each callable raises
        on a non-zero status.

        With ``branch_stream`` (a torch stream) the attention branch (its own mask build, then
        the attention) is enqueued there, everything else on the current stream."""
        lib = L.lib()
        st = torch.cuda.current_stream(self.device).cuda_stream
        fork = branch_stream is not None
        if fork and not self.can_fork():
            raise ValueError("a dynamic tree depends on the heads: the step cannot fork")
        st_b = branch_stream.cuda_stream if fork else st
        calls: Dict[str, Callable[[], None]] = {}
        B, N, D, s_max = self.B, self.N, self.D, self.s_max

        def wrap(name, fn, *args):
            def call():
                r = fn(*args)
                if r != 0:
                    raise L.MVError(name, r)
            return call

        if self.heads is not None:
            hd = self.heads
            d, Vh, K = hd["d"], hd["V"], hd["K"]
            wsp, wsn = self._ws(self.ws_heads)
            calls["heads_residual"] = wrap("mv_medusa_residual", lib.mv_medusa_residual, self.dt, B,
                                           d, K, _p(inp["h"]), _p(inp["w_res"]), None, wsp, wsn, st)
            off = 1 if self.lm_width else 0
            ld = D * s_max
            esz = 4
            proj = wrap("mv_medusa_head_project", lib.mv_medusa_head_project, self.dt, B, d, Vh,
                        K, self._s_heads, s_max, _p(inp["w_head"]),
                        _p(self.draft_logits) if self.spec_lm else None, wsp, wsn, st)
            calls["heads_select"] = wrap("mv_medusa_head_select", lib.mv_medusa_head_select,
                                         self.dt, B, d, Vh, K, self._s_heads, s_max,
                                         self.cand.data_ptr() + off * s_max * esz,
                                         self.cand_vals.data_ptr() + off * s_max * esz, ld,
                                         _p(self.head_lse), wsp, wsn, st)
            if self.lm_width:
                tgt = inp["target"]
                R1, Vt = tgt.shape[1], tgt.shape[2]
                lm = wrap("mv_topk_rows", lib.mv_topk_rows, self.dt, B, Vt, self.lm_width, _p(tgt),
                          R1 * Vt, self.cand.data_ptr(), self.cand_vals.data_ptr(), ld, None, st)

                def both():
                    lm()
                    proj()
                calls["heads_projection"] = both
            else:
                calls["heads_projection"] = proj
        if self.draft_input:
            dl = inp["draft_logits"]
            calls["heads_select"] = wrap("mv_topk_rows", lib.mv_topk_rows, self.dt, B * D, self.V,
                                         s_max, _p(dl), self.V, _p(self.cand),
                                         _p(self.cand_vals), s_max, _p(self.head_lse), st)
        if self.tokens_given:
            calls["tree"] = wrap("mv_build_tree_mask", lib.mv_build_tree_mask, N, _p(self.parents),
                                 0, 0, 0, None, None, _p(self.tree["anc_mask"]),
                                 _p(self.tree["depth"]), None, _p(self.status), st)
            tokens = inp.get("node_tokens")
        elif self.dynamic:
            calls["tree"] = wrap("mv_build_dynamic_tree", lib.mv_build_dynamic_tree, B, D, s_max,
                                 self._s_depth, N, _p(self.cand), _p(self.cand_vals),
                                 _p(self.head_lse), _p(self.parents), _p(self.tree["depth"]),
                                 _p(self.tree["node_tokens"]), _p(self.tree["anc_mask"]),
                                 _p(self.tree["node_logp"]), _p(self.status), st)
            tokens = self.tree["node_tokens"]
        else:
            calls["tree"] = wrap("mv_build_tree_mask", lib.mv_build_tree_mask, N, _p(self.parents),
                                 B, D, s_max, self._s_depth, _p(self.cand),
                                 _p(self.tree["anc_mask"]), _p(self.tree["depth"]),
                                 _p(self.tree["node_tokens"]), _p(self.status), st)
            tokens = self.tree["node_tokens"]
        wsp, wsn = self._ws(self.ws_attn)
        Lcap = inp["k_cache"].shape[2]
        anc = self.tree["anc_mask"]
        if fork:
            anc = self.attn_anc
            calls["attn_mask"] = wrap("mv_build_tree_mask", lib.mv_build_tree_mask, N,
                                      _p(self.parents), 0, 0, 0, None, None, _p(anc), None, None,
                                      _p(self.status), st_b)
        # forked: the launch on half of the CUs (one persistent 8-wave workgroup per CU), so
        # that the bandwidth-bound heads stream their weights on the other half meanwhile
        aname = "mv_tree_attn_verify_beside" if fork else "mv_tree_attn_verify"
        calls["attention"] = wrap(aname, getattr(lib, aname), self.dt, B, N,
                                  self.Hq, self.Hkv, self.dh, Lcap, self.max_L, _p(inp["q"]),
                                  _p(inp["k_cache"]), _p(inp["v_cache"]), _p(inp["prefix_len"]),
                                  _p(anc), N * ((N + 31) // 32) if self.dynamic else 0, 0.0,
                                  _p(self.attn_out),
                                  _p(self.attn_lse), _p(self.status), wsp, wsn, st_b)
        if self.target_head:
            wsp, wsn = self._ws(self.ws_lm)
            calls["target_head"] = wrap("mv_lm_head_argmax", lib.mv_lm_head_argmax, L.MV_BF16,
                                        B * (N + 1), self.target_head, self.V, _p(inp["x_t"]),
                                        _p(inp["w_lm"]), self.target_ids.data_ptr(), None,
                                        _p(self.target_lse) if self.spec_lm else None,
                                        wsp, wsn, st)
        if self.spec_lm:
            wsp, wsn = self._ws(self.ws_accept)
            a = self.acc
            calls["accept"] = wrap("mv_accept_speculative_lm", lib.mv_accept_speculative_lm,
                                   self.dt, B, N, self.V, self.target_head, D, _p(self.parents),
                                   0, _p(tokens), _p(inp["x_t"]), _p(inp["w_lm"]),
                                   _p(self.target_lse),
                                   _p(inp["draft_logits"] if self.draft_input else self.draft_logits),
                                   _p(self.head_lse),
                                   _p(inp["uniforms"]), _p(a["accept_len"]), _p(a["path_nodes"]),
                                   _p(a["out_tokens"]), _p(a["node_accept"]), _p(a["alpha"]),
                                   _p(self.status), wsp, wsn, st)
        elif self.accept != "none":
            wsp, wsn = self._ws(self.ws_accept)
            if self.target_head:
                tgt, tdt, Vt = self.target_ids, L.MV_TARGET_IDS, self.V
            else:
                tgt = inp["target"]
                tdt = L.MV_BF16 if tgt.dtype == torch.bfloat16 else L.MV_F32
                Vt = tgt.shape[2]
            a = self.acc
            calls["accept"] = wrap("mv_accept_paths", lib.mv_accept_paths, self.mode, tdt, B, N,
                                   Vt, D, _p(self.parents), N if self.dynamic else 0, _p(tokens),
                                   _p(tgt),
                                   _p(inp.get("draft")), _p(inp.get("uniforms")),
                                   _p(a["accept_len"]), _p(a["path_nodes"]), _p(a["out_tokens"]),
                                   _p(a["node_accept"]), _p(a["alpha"]), _p(self.status), wsp,
                                   wsn, st)
        if self.commit:
            a = self.acc
            calls["commit"] = wrap("mv_kv_commit", lib.mv_kv_commit, self.dt, B, self.Hkv,
                                   self.dh, Lcap, N, D, _p(inp["k_cache"]), _p(inp["v_cache"]),
                                   _p(inp["prefix_len"]), _p(self.prefix_next),
                                   _p(a["path_nodes"]), _p(a["accept_len"]), _p(self.status), st)
        return calls

    def sequence(self, calls: Dict[str, Callable[[], None]]) -> List[Callable[[], None]]:
        return [calls[p] for p in self.PARTS if p in calls]

    def run(self, inp: Dict[str, torch.Tensor], branch_stream=None) -> None:
        """One whole step on ``inp`` (binds, then runs its calls in order).  With
        ``branch_stream`` (a torch stream) it runs forked, as ``capture(fork=True)`` records it:
        the attention branch on that stream, with the attention launch on half of the CUs."""
        if branch_stream is not None and self.can_fork():
            self._run_forked(inp, branch_stream)
            return
        for c in self.sequence(self.bind(inp)):
            c()

    def _run_forked(self, inp: Dict[str, torch.Tensor], side: "torch.cuda.Stream") -> None:
        """One step with the attention branch on ``side``: it forks from the current stream at
        the start and joins before the commit, which moves K/V rows the attention reads.  The
        acceptance reads only the tree, the target and the draft, so it runs on the main stream
        while the attention may still be running (the attention's outputs are not its input in
        this path; the device status word is OR-ed atomically by both)."""
        main = torch.cuda.current_stream(self.device)
        calls = self.bind(inp, branch_stream=side)
        side.wait_stream(main)
        # the main branch's first call is enqueued ahead of the attention branch, so that a
        # graph of the step starts it first (the heads' chain is the longer branch)
        first = next((n for n in self.PARTS if n not in self.BRANCH and n in calls), None)
        if first is not None:
            calls[first]()
        for name in self.BRANCH:
            calls[name]()
        joined = False
        for name in self.PARTS:
            if name in self.BRANCH or name not in calls or name == first:
                continue
            if name == "commit" and not joined:
                main.wait_stream(side)
                joined = True
            calls[name]()
        if not joined:
            main.wait_stream(side)

    def capture(self, inp: Dict[str, torch.Tensor], fork: bool = False) -> "torch.cuda.CUDAGraph":
        """A HIP graph of one whole step on ``inp`` (replay with ``graph.replay()``).

        The calls are bound inside the capture so that they are enqueued on the capture
        stream; the step allocates nothing and issues no memset, so every replay repeats
        exactly the kernels of an eager step on the same buffers.  With ``fork=True`` the
        attention branch is a parallel branch of the graph beside the heads and the tree."""
        if fork and not self.can_fork():
            fork = False
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream(device=self.device)
        side = torch.cuda.Stream(device=self.device) if fork else None
        s.wait_stream(torch.cuda.current_stream(self.device))
        with torch.cuda.stream(s):       # warm-up on the side stream
            if fork:
                self._run_forked(inp, side)
            else:
                for c in self.sequence(self.bind(inp)):
                    c()
        torch.cuda.current_stream(self.device).wait_stream(s)
        torch.cuda.synchronize(self.device)
        with torch.cuda.graph(g):
            if fork:
                self._run_forked(inp, side)
            else:
                for c in self.sequence(self.bind(inp)):
                    c()
        return g
