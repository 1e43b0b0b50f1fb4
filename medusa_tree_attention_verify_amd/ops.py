"""PyTorch-facing wrappers of the C ABI (argument marshalling only).

Tensors must live on the current HIP device; every call enqueues work on torch's current
stream and returns.  Each function mirrors the C entry point of the same name; see
include/medusa_verify.h for the semantics and the page sections they follow.
"""
from __future__ import annotations

from typing import Dict, Optional, Sequence

import torch

from . import _lib as L

_DT = {torch.float32: L.MV_F32, torch.bfloat16: L.MV_BF16}


def _dt(t: torch.Tensor) -> int:
    if t.dtype not in _DT:
        raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")
    return _DT[t.dtype]


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _need(t: torch.Tensor, name: str, dtype=None, shape=None) -> None:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


class Workspace:
    """Grow-only device scratch buffer handed to the library (256-byte aligned by torch)."""

    def __init__(self, device=None):
        self.device = device
        self.buf: Optional[torch.Tensor] = None

    def get(self, nbytes: int):
        if nbytes == 0:
            return None, 0
        if self.buf is None or self.buf.numel() < nbytes:
            self.buf = torch.empty(nbytes, dtype=torch.uint8, device=self.device or "cuda")
        return self.buf.data_ptr(), self.buf.numel()


_default_ws: Dict[str, Workspace] = {}


def _ws(key: str, ws: Optional[Workspace]) -> Workspace:
    if ws is not None:
        return ws
    if key not in _default_ws:
        _default_ws[key] = Workspace()
    return _default_ws[key]


def device_check(device: int = 0) -> int:
    return L.lib().mv_device_check(int(device))


def validate_parents(parents: Sequence[int]) -> None:
    """Host check of a tree spec: topological parent array with -1 roots."""
    n = len(parents)
    if n < 1 or n > L.MV_MAX_NODES:
        raise ValueError(f"tree must have 1..{L.MV_MAX_NODES} nodes, got {n}")
    for i, p in enumerate(parents):
        if not (-1 <= int(p) < i):
            raise ValueError(f"node {i}: parent {p} is not in [-1, {i})")


# ------------------------------------------------------------------ Medusa heads
def heads_workspace_bytes(dt: int, B: int, d: int, V: int, K: int, s_max: int) -> int:
    return int(L.lib().mv_medusa_heads_workspace(dt, B, d, V, K, s_max))


def medusa_residual(h: torch.Tensor, w_res: torch.Tensor, hk: Optional[torch.Tensor] = None,
                    V: int = 1, s_max: int = 1, ws: Optional[Workspace] = None) -> Workspace:
    """a1: h_k = SiLU(W_res^(k) h) + h.  Returns the workspace holding h_k for the projection."""
    dt = _dt(h)
    B, d = h.shape
    K = w_res.shape[0]
    _need(h, "h")
    _need(w_res, "w_res", h.dtype, (K, d, d))
    if hk is not None:
        _need(hk, "hk", torch.float32, (B, K, d))
    w = _ws("heads", ws)
    ptr, n = w.get(heads_workspace_bytes(dt, B, d, V, K, s_max))
    L.check("mv_medusa_residual", L.lib().mv_medusa_residual(
        dt, B, d, K, _ptr(h), _ptr(w_res), _ptr(hk), ptr, n, _stream()))
    return w


def medusa_head_topk(w_head: torch.Tensor, B: int, s_per_head: Sequence[int],
                     s_max: Optional[int] = None, logits: Optional[torch.Tensor] = None,
                     topk_ids: Optional[torch.Tensor] = None,
                     topk_vals: Optional[torch.Tensor] = None, ld_topk: int = 0,
                     lse: Optional[torch.Tensor] = None,
                     ws: Optional[Workspace] = None) -> Dict[str, torch.Tensor]:
    """a2: logits_k = W_head^(k) h_k (h_k from medusa_residual's workspace), top-s_k, lse.

    Two C calls: mv_medusa_head_project (the weight stream) and mv_medusa_head_select."""
    dt = _dt(w_head)
    K, V, d = w_head.shape
    s_max = int(s_max or max(s_per_head))
    _need(w_head, "w_head")
    dev = w_head.device
    if topk_ids is None:
        topk_ids = torch.empty((B, K, s_max), dtype=torch.int32, device=dev)
    if topk_vals is None:
        topk_vals = torch.empty(topk_ids.shape, dtype=torch.float32, device=dev)
    if logits is not None:
        _need(logits, "logits", w_head.dtype, (B, K, V))
    if lse is not None:
        _need(lse, "lse", torch.float32, (B, K))
    w = _ws("heads", ws)
    ptr, n = w.get(heads_workspace_bytes(dt, B, d, V, K, s_max))
    sp = L.int_array(s_per_head)
    L.check("mv_medusa_head_project", L.lib().mv_medusa_head_project(
        dt, B, d, V, K, sp, s_max, _ptr(w_head), _ptr(logits), ptr, n, _stream()))
    L.check("mv_medusa_head_select", L.lib().mv_medusa_head_select(
        dt, B, d, V, K, sp, s_max, _ptr(topk_ids), _ptr(topk_vals), int(ld_topk), _ptr(lse),
        ptr, n, _stream()))
    return {"topk_ids": topk_ids, "topk_vals": topk_vals, "logits": logits, "lse": lse}


def medusa_heads(h: torch.Tensor, w_res: torch.Tensor, w_head: torch.Tensor,
                 s_per_head: Sequence[int], s_max: Optional[int] = None, want_hk: bool = False,
                 want_logits: bool = False, want_lse: bool = True,
                 ws: Optional[Workspace] = None) -> Dict[str, torch.Tensor]:
    """a1 + a2 in one call."""
    dt = _dt(h)
    B, d = h.shape
    K, V, _ = w_head.shape
    s_max = int(s_max or max(s_per_head))
    for t, nm in ((h, "h"), (w_res, "w_res"), (w_head, "w_head")):
        _need(t, nm, h.dtype)
    dev = h.device
    hk = torch.empty((B, K, d), dtype=torch.float32, device=dev) if want_hk else None
    logits = torch.empty((B, K, V), dtype=h.dtype, device=dev) if want_logits else None
    lse = torch.empty((B, K), dtype=torch.float32, device=dev) if want_lse else None
    ids = torch.empty((B, K, s_max), dtype=torch.int32, device=dev)
    vals = torch.empty((B, K, s_max), dtype=torch.float32, device=dev)
    w = _ws("heads", ws)
    ptr, n = w.get(heads_workspace_bytes(dt, B, d, V, K, s_max))
    L.check("mv_medusa_heads", L.lib().mv_medusa_heads(
        dt, B, d, V, K, L.int_array(s_per_head), s_max, _ptr(h), _ptr(w_res), _ptr(w_head),
        _ptr(hk), _ptr(logits), _ptr(ids), _ptr(vals), 0, _ptr(lse), ptr, n, _stream()))
    return {"hk": hk, "logits": logits, "topk_ids": ids, "topk_vals": vals, "lse": lse}


def topk_rows(x: torch.Tensor, s: int, R: Optional[int] = None, V: Optional[int] = None,
              ldx: Optional[int] = None, ids: Optional[torch.Tensor] = None,
              vals: Optional[torch.Tensor] = None, ld_out: Optional[int] = None,
              lse: Optional[torch.Tensor] = None):
    """Top-s of R rows of x (row r at r*ldx elements), and each row's log-sum-exp into ``lse``
    (fp32 [R]) when given.  Defaults: x is [R, V] contiguous."""
    dt = _dt(x)
    if R is None or V is None:
        R, V = x.shape[-2], x.shape[-1]
    ldx = V if ldx is None else ldx
    if ids is None:
        ids = torch.empty((R, s), dtype=torch.int32, device=x.device)
        vals = torch.empty((R, s), dtype=torch.float32, device=x.device) if vals is None else vals
        ld_out = s
    L.check("mv_topk_rows", L.lib().mv_topk_rows(dt, R, V, s, _ptr(x), int(ldx), _ptr(ids),
                                                 _ptr(vals), int(ld_out or s), _ptr(lse),
                                                 _stream()))
    return ids, vals


# ------------------------------------------------------------------ tree
def build_tree_mask(parents: torch.Tensor, cand: Optional[torch.Tensor] = None,
                    s_per_depth: Optional[Sequence[int]] = None,
                    status: Optional[torch.Tensor] = None,
                    out: Optional[Dict[str, torch.Tensor]] = None) -> Dict[str, torch.Tensor]:
    """a3: parents [N] int32 -> anc_mask [N, ceil(N/32)] uint32 (as int32), depth, node_tokens."""
    _need(parents, "parents", torch.int32)
    N = parents.numel()
    W = (N + 31) // 32
    dev = parents.device
    B = D = s_max = 0
    if cand is not None:
        _need(cand, "cand", torch.int32)
        B, D, s_max = cand.shape
    if out is None:
        out = {"anc_mask": torch.empty((N, W), dtype=torch.int32, device=dev),
               "depth": torch.empty(N, dtype=torch.int32, device=dev),
               "node_tokens": torch.empty((B, N), dtype=torch.int32, device=dev)
               if cand is not None else None}
    sp = L.int_array(s_per_depth) if s_per_depth is not None else None
    L.check("mv_build_tree_mask", L.lib().mv_build_tree_mask(
        N, _ptr(parents), B, D, s_max, sp, _ptr(cand), _ptr(out["anc_mask"]), _ptr(out["depth"]),
        _ptr(out.get("node_tokens")), _ptr(status), _stream()))
    return out


def build_dynamic_tree(cand_ids: torch.Tensor, cand_vals: torch.Tensor,
                       cand_lse: Optional[torch.Tensor], N: int,
                       s_per_depth: Optional[Sequence[int]] = None,
                       status: Optional[torch.Tensor] = None,
                       out: Optional[Dict[str, torch.Tensor]] = None) -> Dict[str, torch.Tensor]:
    """Per-sequence tree of the N most probable candidate paths.  cand_ids int32 and
    cand_vals fp32 [B, D, s_max] (best first), cand_lse fp32 [B, D] or None (values are
    log-probabilities).  Returns parents, depth, node_tokens [B, N], anc_mask [B, N, W] (as
    int32), node_logp [B, N]."""
    B, D, s_max = cand_ids.shape
    _need(cand_ids, "cand_ids", torch.int32)
    _need(cand_vals, "cand_vals", torch.float32, (B, D, s_max))
    if cand_lse is not None:
        _need(cand_lse, "cand_lse", torch.float32, (B, D))
    W = (N + 31) // 32
    dev = cand_ids.device
    if out is None:
        out = {"parents": torch.empty((B, N), dtype=torch.int32, device=dev),
               "depth": torch.empty((B, N), dtype=torch.int32, device=dev),
               "node_tokens": torch.empty((B, N), dtype=torch.int32, device=dev),
               "anc_mask": torch.empty((B, N, W), dtype=torch.int32, device=dev),
               "node_logp": torch.empty((B, N), dtype=torch.float32, device=dev)}
    sp = L.int_array(s_per_depth) if s_per_depth is not None else None
    L.check("mv_build_dynamic_tree", L.lib().mv_build_dynamic_tree(
        B, D, s_max, sp, N, _ptr(cand_ids), _ptr(cand_vals), _ptr(cand_lse),
        _ptr(out["parents"]), _ptr(out["depth"]), _ptr(out["node_tokens"]), _ptr(out["anc_mask"]),
        _ptr(out.get("node_logp")), _ptr(status), _stream()))
    return out


# ------------------------------------------------------------------ attention
def attn_workspace_bytes(dt: int, B: int, N: int, Hq: int, Hkv: int, dh: int, max_L: int,
                         beside: bool = False) -> int:
    fn = L.lib().mv_tree_attn_verify_beside_workspace if beside else L.lib().mv_tree_attn_verify_workspace
    return int(fn(dt, B, N, Hq, Hkv, dh, max_L))


def tree_attn_verify(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                     prefix_len: torch.Tensor, anc_mask: torch.Tensor, max_L: int,
                     scale: float = 0.0, out: Optional[torch.Tensor] = None,
                     lse: Optional[torch.Tensor] = None, want_lse: bool = True,
                     status: Optional[torch.Tensor] = None,
                     ws: Optional[Workspace] = None, beside: bool = False):
    """a4 + a5: tree-masked GQA attention; returns (out [B,N,Hq,dh], lse [B,Hq,N] or None).

    anc_mask [N, W] (one tree for the batch) or [B, N, W] (one tree per sequence).
    ``beside`` takes the launch on half of the CUs (mv_tree_attn_verify_beside), meant to run
    on one stream while bandwidth-bound kernels run on another."""
    dt = _dt(q)
    B, N, Hq, dh = q.shape
    _, Hkv, L_cap, _ = k_cache.shape
    _need(q, "q")
    _need(k_cache, "k_cache", q.dtype, (B, Hkv, L_cap, dh))
    _need(v_cache, "v_cache", q.dtype, (B, Hkv, L_cap, dh))
    _need(prefix_len, "prefix_len", torch.int32, (B,))
    W = (N + 31) // 32
    if anc_mask.dim() == 3:
        _need(anc_mask, "anc_mask", None, (B, N, W))
        mstride = N * W
    else:
        _need(anc_mask, "anc_mask", None, (N, W))
        mstride = 0
    if out is None:
        out = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device)
    w = _ws("attn", ws)
    ptr, n = w.get(attn_workspace_bytes(dt, B, N, Hq, Hkv, dh, max_L, beside))
    name = "mv_tree_attn_verify_beside" if beside else "mv_tree_attn_verify"
    L.check(name, getattr(L.lib(), name)(
        dt, B, N, Hq, Hkv, dh, L_cap, int(max_L), _ptr(q), _ptr(k_cache), _ptr(v_cache),
        _ptr(prefix_len), _ptr(anc_mask), mstride, float(scale), _ptr(out), _ptr(lse),
        _ptr(status),
        ptr, n, _stream()))
    return out, lse


# ------------------------------------------------------------------ acceptance
def accept_workspace_bytes(mode: int, B: int, N: int, V: int) -> int:
    return int(L.lib().mv_accept_paths_workspace(mode, B, N, V))


def lm_head_workspace_bytes(T: int, d: int, V: int) -> int:
    return int(L.lib().mv_lm_head_workspace(L.MV_BF16, T, d, V))


def lm_head_argmax(x: torch.Tensor, w_lm: torch.Tensor, want_max: bool = True,
                   want_lse: bool = True, out: Optional[Dict[str, torch.Tensor]] = None,
                   ws: Optional[Workspace] = None) -> Dict[str, torch.Tensor]:
    """Target LM head over T rows of hidden states x [T, d] (bf16) with W [V, d] (bf16): the
    greedy token per row (int32), and optionally its logit and the row's LSE (fp32)."""
    _need(x, "x", torch.bfloat16)
    _need(w_lm, "w_lm", torch.bfloat16)
    T, d = x.shape
    V, d2 = w_lm.shape
    if d2 != d:
        raise ValueError(f"w_lm is [V, {d2}] but x has d = {d}")
    dev = x.device
    if out is None:
        out = {"ids": torch.empty(T, dtype=torch.int32, device=dev),
               "max": torch.empty(T, dtype=torch.float32, device=dev) if want_max else None,
               "lse": torch.empty(T, dtype=torch.float32, device=dev) if want_lse else None}
    w = _ws("lm_head", ws)
    ptr, n = w.get(lm_head_workspace_bytes(T, d, V))
    L.check("mv_lm_head_argmax", L.lib().mv_lm_head_argmax(
        L.MV_BF16, T, d, V, _ptr(x), _ptr(w_lm), _ptr(out["ids"]), _ptr(out.get("max")),
        _ptr(out.get("lse")), ptr, n, _stream()))
    return out


def accept_paths(mode: int, parents: torch.Tensor, node_tokens: torch.Tensor,
                 target: torch.Tensor, D: int, draft: Optional[torch.Tensor] = None,
                 uniforms: Optional[torch.Tensor] = None, want_node_accept: bool = True,
                 want_alpha: bool = True, status: Optional[torch.Tensor] = None,
                 out: Optional[Dict[str, torch.Tensor]] = None,
                 ws: Optional[Workspace] = None, vocab: Optional[int] = None) -> Dict[str, torch.Tensor]:
    """a6 (greedy) / a7 (speculative) / multi-candidate (siblings tested in turn against the
    running residual): accepted length, path, committed tokens + extra token.

    Greedy also takes the target rows as argmax ids: target int32 [B, N+1] (then V = vocab
    size must be given, used only to range-check node tokens).  parents [N] (one tree for the
    batch) or [B, N] (one tree per sequence)."""
    if target.dtype == torch.int32:
        if mode != L.MV_ACCEPT_GREEDY or vocab is None:
            raise ValueError("argmax-id targets need greedy mode and vocab=")
        dt = L.MV_TARGET_IDS
        B, R = target.shape
        V = int(vocab)
    else:
        dt = _dt(target)
        B, R, V = target.shape
    N = R - 1
    if parents.dim() == 2:
        _need(parents, "parents", torch.int32, (B, N))
        pstride = N
    else:
        _need(parents, "parents", torch.int32, (N,))
        pstride = 0
    _need(node_tokens, "node_tokens", torch.int32, (B, N))
    _need(target, "target")
    spec = mode in (L.MV_ACCEPT_SPECULATIVE, L.MV_ACCEPT_MULTICAND)
    if spec:
        _need(draft, "draft", torch.float32, (B, R, V))
        _need(uniforms, "uniforms", torch.float32, (B, R))
    dev = target.device
    if out is None:
        out = {"accept_len": torch.empty(B, dtype=torch.int32, device=dev),
               "path_nodes": torch.empty((B, D), dtype=torch.int32, device=dev),
               "out_tokens": torch.empty((B, D + 1), dtype=torch.int32, device=dev),
               "node_accept": torch.empty((B, N), dtype=torch.uint8, device=dev)
               if want_node_accept else None,
               "alpha": torch.empty((B, N), dtype=torch.float32, device=dev)
               if (want_alpha and spec) else None}
    w = _ws("accept", ws)
    ptr, n = (None, 0) if dt == L.MV_TARGET_IDS else w.get(accept_workspace_bytes(mode, B, N, V))
    L.check("mv_accept_paths", L.lib().mv_accept_paths(
        mode, dt, B, N, V, D, _ptr(parents), pstride, _ptr(node_tokens), _ptr(target), _ptr(draft),
        _ptr(uniforms), _ptr(out["accept_len"]), _ptr(out["path_nodes"]), _ptr(out["out_tokens"]),
        _ptr(out.get("node_accept")), _ptr(out.get("alpha")), _ptr(status), ptr, n, _stream()))
    return out


def accept_speculative_lm(parents: torch.Tensor, node_tokens: torch.Tensor, x_t: torch.Tensor,
                          w_lm: torch.Tensor, lse_t: torch.Tensor, draft_logits: torch.Tensor,
                          draft_lse: torch.Tensor, uniforms: torch.Tensor, D: int,
                          status: Optional[torch.Tensor] = None,
                          out: Optional[Dict[str, torch.Tensor]] = None,
                          ws: Optional[Workspace] = None) -> Dict[str, torch.Tensor]:
    """Speculative acceptance with the target from the LM head (x_t [B, N+1, d] bf16, w_lm
    [V, d] bf16, lse_t [B, N+1]) and the draft from per-depth logits (draft_logits [B, D, V]
    fp32 or bf16, draft_lse [B, D]); no [B, N+1, V] probabilities."""
    B, R, d = x_t.shape
    N = R - 1
    V = w_lm.shape[0]
    if parents.dim() == 2:
        _need(parents, "parents", torch.int32, (B, N))
        pstride = N
    else:
        _need(parents, "parents", torch.int32, (N,))
        pstride = 0
    _need(node_tokens, "node_tokens", torch.int32, (B, N))
    _need(x_t, "x_t", torch.bfloat16, (B, R, d))
    _need(w_lm, "w_lm", torch.bfloat16, (V, d))
    _need(lse_t, "lse_t", torch.float32, (B, R))
    _need(draft_logits, "draft_logits", None, (B, D, V))
    _need(draft_lse, "draft_lse", torch.float32, (B, D))
    _need(uniforms, "uniforms", torch.float32, (B, R))
    ddt = _dt(draft_logits)
    dev = x_t.device
    if out is None:
        out = {"accept_len": torch.empty(B, dtype=torch.int32, device=dev),
               "path_nodes": torch.empty((B, D), dtype=torch.int32, device=dev),
               "out_tokens": torch.empty((B, D + 1), dtype=torch.int32, device=dev),
               "node_accept": torch.empty((B, N), dtype=torch.uint8, device=dev),
               "alpha": torch.empty((B, N), dtype=torch.float32, device=dev)}
    w = _ws("accept_lm", ws)
    ptr, n = w.get(L.lib().mv_accept_speculative_lm_workspace(B, N, V))
    L.check("mv_accept_speculative_lm", L.lib().mv_accept_speculative_lm(
        ddt, B, N, V, d, D, _ptr(parents), pstride, _ptr(node_tokens), _ptr(x_t), _ptr(w_lm),
        _ptr(lse_t), _ptr(draft_logits), _ptr(draft_lse), _ptr(uniforms),
        _ptr(out["accept_len"]), _ptr(out["path_nodes"]), _ptr(out["out_tokens"]),
        _ptr(out.get("node_accept")), _ptr(out.get("alpha")), _ptr(status), ptr, n, _stream()))
    return out


def kv_commit(k_cache: torch.Tensor, v_cache: torch.Tensor, prefix_len: torch.Tensor, N: int,
              path_nodes: torch.Tensor, accept_len: torch.Tensor,
              status: Optional[torch.Tensor] = None,
              prefix_out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Move the accepted path's K/V rows L+path[j] -> L+j (all KV heads, in place) and write
    prefix_len + accept_len to prefix_out (default: prefix_len itself).  Returns prefix_out."""
    dt = _dt(k_cache)
    B, Hkv, L_cap, dh = k_cache.shape
    _need(k_cache, "k_cache")
    _need(v_cache, "v_cache", k_cache.dtype, tuple(k_cache.shape))
    _need(prefix_len, "prefix_len", torch.int32, (B,))
    D = path_nodes.shape[1]
    _need(path_nodes, "path_nodes", torch.int32, (B, D))
    _need(accept_len, "accept_len", torch.int32, (B,))
    if prefix_out is None:
        prefix_out = prefix_len
    _need(prefix_out, "prefix_out", torch.int32, (B,))
    L.check("mv_kv_commit", L.lib().mv_kv_commit(
        dt, B, Hkv, dh, L_cap, N, D, _ptr(k_cache), _ptr(v_cache), _ptr(prefix_len),
        _ptr(prefix_out), _ptr(path_nodes), _ptr(accept_len), _ptr(status), _stream()))
    return prefix_out
