"""CPU oracle for the Medusa single-pass tree verification step.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import or call
this module: only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline
leg of ``bench.py`` use it.  It shares no code with the HIP library.

Every function is the plain definition of what the step computes, in float64
(inputs are upcast exactly), with no blocking, online softmax, splitting or
fusion.  Sources (web pages on Medusa and tree-structured speculative
verification):

* "Medusa Explained: Multi-Head Speculative Decoding Guide" (aifetchly blog):
  section "The Architectural Blueprint" (residual-block and softmax
  equations of a Medusa head), "1. Combinatorial Tree Construction",
  "2. Single-Pass Tree Attention Verification" (additive mask M_tree and the
  5-candidate mask example, greedy longest-accepted-path rule).
* "Multi-Token Prediction: Draft-Model-Free Speculative Decoding"
  (globaltechdigest blog): "The 2D Tree Attention Mask" (boolean mask,
  ancestor-or-self), the verification-engine code (a parent array with -1
  roots; the committed path is the longest accepted one, the first of equal
  ones) and the text box of Figure 1 (the target adds one token after the
  committed path), and
  "Production Deployment Guidelines" (unselected branches culled from the KV
  cache after verification).
* "Speculative Decoding & Medusa Tree Attention" (akmalkhaniub blog):
  section 2, "The Acceptance Sampling Rule" (alpha = min(1, P_t/P_d) and the
  residual distribution normalize(max(0, P_t - P_d)); P_target is the softmax of
  the target model's logits).

Readings where the pages are silent (scale 1/sqrt(dh), contiguous GQA groups,
tree K/V appended after the prefix, ties, the speculative rule applied node by
node, sampling by inverse CDF) are stated next to the code that takes them.

Parity pins: every function here is pinned by tests under ``tests/`` against
worked examples printed on the pages, closed forms, invariants and brute-force
references; none is "parity unpinned".
"""
from __future__ import annotations

from typing import Dict, List, Optional, Sequence

import numpy as np

__all__ = [
    "silu", "medusa_heads", "topk_rows", "build_tree", "tree_attention",
    "accept_greedy", "accept_speculative", "paths_to_parents", "lm_head_argmax", "kv_commit",
    "accept_multicandidate", "dynamic_tree", "accept_speculative_lm",
]


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


# --------------------------------------------------------------------------
# 1. Medusa heads  ("The Architectural Blueprint", residual-block equation)
# --------------------------------------------------------------------------
def silu(x: np.ndarray) -> np.ndarray:
    """SiLU(x) = x * sigmoid(x) = x / (1 + exp(-x))."""
    x = _f64(x)
    with np.errstate(over="ignore"):
        return x / (1.0 + np.exp(-x))


def topk_rows(rows: np.ndarray, s: int) -> Dict[str, np.ndarray]:
    """Top-s entries of each row: larger value first, equal values by lower index.

    The order is a stable sort on (-value, index); returns ids (int64) and values.
    """
    rows = _f64(rows)
    order = np.argsort(-rows, axis=-1, kind="stable")[..., :s]
    return {"ids": order.astype(np.int64), "vals": np.take_along_axis(rows, order, axis=-1)}


def medusa_heads(h, w_res, w_head, widths: Sequence[int]) -> Dict[str, np.ndarray]:
    """Medusa heads for a batch of hidden states.

    For head k:  u = W_res[k] h,  h_k = SiLU(u) + h,  logits_k = W_head[k] h_k
    (the residual block has no bias, as in the page's equation), and
    p_k = softmax(logits_k).  Head k's candidates are its top-``widths[k]``
    logits (softmax is monotone, so the top of p_k is the top of logits_k).

    Shapes: h [B,d]; w_res [K,d,d] stored (out, in); w_head [K,V,d].
    Returns hk [B,K,d], logits [B,K,V], topk_ids/topk_vals [B,K,s_max]
    (-1 / -inf padded past widths[k]), lse [B,K] = log sum exp(logits).
    """
    h = _f64(h)
    B, d = h.shape
    K, V, _ = np.shape(w_head)
    s_max = max(widths)
    hk = np.empty((B, K, d))
    logits = np.empty((B, K, V))
    ids = np.full((B, K, s_max), -1, dtype=np.int64)
    vals = np.full((B, K, s_max), -np.inf)
    lse = np.empty((B, K))
    for k in range(K):
        wr, wh = _f64(w_res[k]), _f64(w_head[k])   # one head at a time in host memory
        for b in range(B):
            u = wr @ h[b]
            hk[b, k] = silu(u) + h[b]
            z = wh @ hk[b, k]
            logits[b, k] = z
            t = topk_rows(z, widths[k])
            ids[b, k, :widths[k]] = t["ids"]
            vals[b, k, :widths[k]] = t["vals"]
            m = z.max()
            lse[b, k] = m + np.log(np.exp(z - m).sum())
    return {"hk": hk, "logits": logits, "topk_ids": ids, "topk_vals": vals, "lse": lse}


# --------------------------------------------------------------------------
# 2. Tree assembly  ("1. Combinatorial Tree Construction"; the boolean
#    ancestor-or-self mask of "The 2D Tree Attention Mask"; the parent-array
#    walk of the verification-engine code)
# --------------------------------------------------------------------------
def paths_to_parents(paths: Sequence[Sequence[int]]):
    """Convert root-to-node paths of node labels into (labels, parent array).

    A label becomes a node the first time it is seen (in path order); its
    parent is the previous label on that path, or -1 at the head of a path.
    """
    labels: List[int] = []
    index: Dict[int, int] = {}
    parents: List[int] = []
    for path in paths:
        prev = -1
        for lab in path:
            if lab not in index:
                index[lab] = len(labels)
                labels.append(lab)
                parents.append(prev)
            prev = index[lab]
    return labels, parents


def build_tree(parents: Sequence[int], cand: Optional[Sequence[np.ndarray]] = None,
               widths: Optional[Sequence[int]] = None) -> Dict[str, object]:
    """Depth, sibling rank, ancestor-or-self sets/bitmask and node tokens.

    parents[i] is the parent of node i, -1 for a node that hangs directly off
    the prefix; the array must be topological (-1 <= parents[i] < i).
    depth[i] = 1 for parent -1, else depth[parent] + 1.  anc[i] = {i} plus
    anc[parent].  rank[i] = number of earlier siblings.  With candidates
    cand[k] ([B, >= s_k] token ids for depth k+1), node i's token is
    cand[depth-1][b, rank], which requires rank < widths[depth-1].
    The bitmask has W = ceil(N/32) uint32 words per node; bit j of word j//32
    of row i is set iff j is in anc[i].
    """
    N = len(parents)
    depth = np.zeros(N, dtype=np.int64)
    rank = np.zeros(N, dtype=np.int64)
    anc: List[List[int]] = []
    for i in range(N):
        p = int(parents[i])
        if not (-1 <= p < i):
            raise ValueError(f"node {i}: parent {p} is not in [-1, {i})")
        depth[i] = 1 if p == -1 else depth[p] + 1
        rank[i] = sum(1 for j in range(i) if int(parents[j]) == p)
        anc.append(sorted(([i] + (anc[p] if p >= 0 else []))))
    W = (N + 31) // 32
    bits = np.zeros((N, W), dtype=np.uint32)
    for i in range(N):
        for j in anc[i]:
            bits[i, j // 32] |= np.uint32(1) << np.uint32(j % 32)
    out: Dict[str, object] = {"depth": depth, "rank": rank, "anc": anc, "mask_bits": bits}
    if cand is not None:
        B = np.asarray(cand[0]).shape[0]
        tokens = np.zeros((B, N), dtype=np.int64)
        for i in range(N):
            k = int(depth[i]) - 1
            if k >= len(cand):
                raise ValueError(f"node {i} at depth {k + 1} has no candidate list")
            w = widths[k] if widths is not None else np.asarray(cand[k]).shape[1]
            if rank[i] >= w:
                raise ValueError(f"node {i}: rank {rank[i]} >= width {w} at depth {k + 1}")
            tokens[:, i] = np.asarray(cand[k])[:, rank[i]]
        out["tokens"] = tokens
    return out


def mask_matrix(anc: Sequence[Sequence[int]]) -> np.ndarray:
    """The ancestor-or-self sets as an N x N boolean matrix (row i is True exactly at the
    columns listed in anc[i])."""
    N = len(anc)
    m = np.zeros((N, N), dtype=bool)
    for i, a in enumerate(anc):
        m[i, list(a)] = True
    return m


# --------------------------------------------------------------------------
# 3. Tree-masked GQA attention ("2. Single-Pass Tree Attention Verification":
#    the tree is packed after the prefix and every node sees the prefix plus
#    its ancestors and itself; additive mask 0 / -inf)
# --------------------------------------------------------------------------
def tree_attention(q, k_cache, v_cache, prefix_len, anc: Sequence[Sequence[int]],
                   scale: Optional[float] = None,
                   select: Optional[Sequence[tuple]] = None) -> Dict[str, np.ndarray]:
    """Scaled dot-product attention of every tree node over prefix + ancestors.

    q [B,N,Hq,dh]; k_cache/v_cache [B,Hkv,L_cap,dh] hold the prefix at rows
    [0, L_b) and the tree's own K/V at rows [L_b, L_b+N) in node order.
    Query head h reads KV head h // (Hq/Hkv).  For node i the visible keys are
    all L_b prefix rows and the rows L_b + j for j in anc[i]; scores are
    q.k * scale (default 1/sqrt(dh)), masked to -inf elsewhere, softmaxed,
    and applied to V.  Returns out [B,N,Hq,dh] and lse [B,Hq,N] (natural log).

    ``select`` = list of (b, h, i) computes only those outputs (others NaN).
    """
    q, k_cache, v_cache = _f64(q), k_cache, v_cache
    B, N, Hq, dh = q.shape
    Hkv = k_cache.shape[1]
    G = Hq // Hkv
    if scale is None or scale <= 0:
        scale = 1.0 / np.sqrt(dh)
    out = np.full((B, N, Hq, dh), np.nan)
    lse = np.full((B, Hq, N), np.nan)
    if select is None:
        select = [(b, h, i) for b in range(B) for h in range(Hq) for i in range(N)]
    todo: Dict[tuple, List[tuple]] = {}
    for b, h, i in select:
        todo.setdefault((b, h // G), []).append((h, i))
    for (b, g), items in todo.items():
        L = int(prefix_len[b])
        keys = _f64(k_cache[b, g, :L + N])
        vals = _f64(v_cache[b, g, :L + N])
        for h, i in items:
            visible = np.zeros(L + N, dtype=bool)
            visible[:L] = True
            visible[[L + j for j in anc[i]]] = True
            s = (keys @ q[b, i, h]) * scale
            s = np.where(visible, s, -np.inf)
            m = s.max()
            e = np.exp(s - m)
            z = e.sum()
            out[b, i, h] = (e @ vals) / z
            lse[b, h, i] = m + np.log(z)
    return {"out": out, "lse": lse}


# --------------------------------------------------------------------------
# 4a. Greedy acceptance ("2. Single-Pass Tree Attention Verification", step 3:
#     the committed path is the longest one on which every token equals the
#     target's greedy choice; the verification-engine code keeps the first of
#     equally long paths; the Figure-1 text box adds one token from the target
#     after the path)
# --------------------------------------------------------------------------
def _committed_path(parents, passes):
    """Accepted nodes and the committed path of one sequence, from each node's own test.

    passes[i] is node i's own test (token match, or u < alpha).  A node is accepted when it
    and every node of its ancestor-or-self set pass, i.e. when the whole chain of candidate
    tokens from the prefix down to it is taken.  The ancestor-or-self set of a node has as
    many members as the node's depth, so among the accepted nodes the committed one is the
    one with the largest set, the lowest node index among equals.  Its path, root first, is
    that set in increasing index order (a parent always has a smaller index than its child).
    Returns (accepted [N] bool, terminal node or -1 for the prefix, path list)."""
    anc = build_tree(parents)["anc"]
    accepted = np.array([all(bool(passes[j]) for j in a) for a in anc], dtype=bool)
    size = np.where(accepted, [len(a) for a in anc], 0)
    if size.size == 0 or size.max() == 0:
        return accepted, -1, []
    term = int(np.flatnonzero(size == size.max())[0])
    return accepted, term, sorted(anc[term])


def _pack(paths_tokens, B, D):
    acc_len = np.zeros(B, dtype=np.int64)
    path_nodes = np.full((B, D), -1, dtype=np.int64)
    out_tokens = np.full((B, D + 1), -1, dtype=np.int64)
    for b, (path, toks, bonus) in enumerate(paths_tokens):
        acc_len[b] = len(path)
        path_nodes[b, :len(path)] = path
        out_tokens[b, :len(path)] = toks
        out_tokens[b, len(path)] = bonus
    return acc_len, path_nodes, out_tokens


def accept_greedy(target, node_tokens, parents, D: int) -> Dict[str, np.ndarray]:
    """Greedy longest-accepted-path acceptance.

    target [B, N+1, V]: row 0 is the distribution after the last prefix token,
    row i+1 the one after node i.  pred[r] = argmax of row r (first index on
    ties).  Node i passes when its token equals pred at its parent's row, and
    is accepted when every node from its root down to it passes.  The
    committed path ends at the deepest accepted node (lowest index on ties);
    the bonus token is pred at that node's row (row 0 if none).
    """
    target = _f64(target)
    B, R, V = target.shape
    N = len(parents)
    pred = np.argmax(target, axis=-1)          # first maximal index
    prow = np.asarray(parents, dtype=np.int64) + 1   # row of each node's parent
    accepted = np.zeros((B, N), dtype=bool)
    res = []
    for b in range(B):
        passes = np.asarray(node_tokens[b], dtype=np.int64) == pred[b, prow]
        accepted[b], term, path = _committed_path(parents, passes)
        res.append((path, [int(node_tokens[b, n]) for n in path], int(pred[b, term + 1])))
    acc_len, path_nodes, out_tokens = _pack(res, B, D)
    return {"accept_len": acc_len, "path_nodes": path_nodes, "out_tokens": out_tokens,
            "node_accept": accepted, "pred": pred}


# --------------------------------------------------------------------------
# 4b. Speculative acceptance ("The Acceptance Sampling Rule": accept x with
#     probability min(1, P_t(x)/P_d(x)), else resample from
#     normalize(max(0, P_t - P_d)); applied node by node on the tree)
# --------------------------------------------------------------------------
def _inverse_cdf(r: np.ndarray, u: float) -> int:
    """First j with cumsum(r)[j] > u * sum(r); the last j with r_j > 0 if none."""
    c = np.cumsum(r)
    t = float(u) * c[-1]
    hit = np.nonzero(c > t)[0]
    if hit.size:
        return int(hit[0])
    pos = np.nonzero(r > 0)[0]
    return int(pos[-1]) if pos.size else len(r) - 1


def accept_speculative(p_target, p_draft, node_tokens, parents, uniforms,
                       D: int) -> Dict[str, np.ndarray]:
    """Speculative (rejection-sampling) acceptance over a candidate tree.

    p_target/p_draft [B, N+1, V] probabilities (row 0 = after the prefix, row
    i+1 = after node i); uniforms [B, N+1] in [0, 1).
    alpha_i = min(1, P_t[parent row, x_i] / P_d[parent row, x_i]) (1 when
    P_d = 0); node i passes iff u[b, i] < alpha_i and is accepted iff every
    node from its root down to it passes.  The path ends at the
    deepest accepted node e (lowest index on ties; e = prefix if none).  The
    extra token is drawn with u[b, N] by inverse CDF from
    normalize(max(0, P_t[e] - P_d[e])) when e has children (all of them were
    rejected), falling back to P_t[e] when that residual is all zero, and
    from P_t[e] when e is a leaf.
    """
    p_t, p_d = _f64(p_target), _f64(p_draft)
    u = _f64(uniforms)
    B, R, V = p_t.shape
    N = len(parents)
    has_child = np.zeros(N + 1, dtype=bool)    # index = row (node + 1); row 0 = prefix
    for i in range(N):
        has_child[int(parents[i]) + 1] = True
    prow = np.asarray(parents, dtype=np.int64) + 1   # row of each node's parent
    alpha = np.zeros((B, N))
    accepted = np.zeros((B, N), dtype=bool)
    res = []
    for b in range(B):
        x = np.asarray(node_tokens[b], dtype=np.int64)
        pt, pd = p_t[b, prow, x], p_d[b, prow, x]
        with np.errstate(divide="ignore", invalid="ignore"):
            alpha[b] = np.where(pd == 0.0, 1.0, np.minimum(1.0, pt / np.where(pd == 0.0, 1.0, pd)))
        accepted[b], term, path = _committed_path(parents, u[b, :N] < alpha[b])
        row = term + 1
        if has_child[row]:
            r = np.maximum(0.0, p_t[b, row] - p_d[b, row])
            if r.sum() <= 0.0:
                r = p_t[b, row]
        else:
            r = p_t[b, row]
        tok = _inverse_cdf(r, u[b, N])
        res.append((path, [int(node_tokens[b, n]) for n in path], tok))
    acc_len, path_nodes, out_tokens = _pack(res, B, D)
    return {"accept_len": acc_len, "path_nodes": path_nodes, "out_tokens": out_tokens,
            "node_accept": accepted, "alpha": alpha}


# --------------------------------------------------------------------------
# 6. Target LM head over the verification rows ("2. Single-Pass Tree Attention
#    Verification", step 2: the target model outputs a distribution for every
#    candidate node, step 3 compares each node with its greedy prediction;
#    "The Acceptance Sampling Rule": P_target = softmax of the logits)
# --------------------------------------------------------------------------
def lm_head_argmax(x, w) -> Dict[str, np.ndarray]:
    """Target logits z[t] = W x[t] for hidden-state rows x [T, d] and the LM-head weight
    W [V, d] (one row per vocabulary entry).  Per row: the greedy token (the first, i.e.
    lowest, index of the maximum), that logit, and LSE = log sum_v exp(z[t][v]), so that
    P_target(v) = exp(z[t][v] - LSE).  Also returns the logits."""
    x, w = _f64(x), _f64(w)
    z = x @ w.T
    ids = np.argmax(z, axis=1)
    mx = z[np.arange(z.shape[0]), ids]
    lse = mx + np.log(np.exp(z - mx[:, None]).sum(axis=1))
    return {"ids": ids.astype(np.int64), "max": mx, "lse": lse, "logits": z}


# --------------------------------------------------------------------------
# 6b. Speculative acceptance with the target from the LM head and the draft
#     from the Medusa heads ("The Acceptance Sampling Rule": P_target is the
#     softmax of the target's logits; "2. Single-Pass Tree Attention
#     Verification", step 2: the target gives a distribution at every
#     candidate node; "The Architectural Blueprint": head k's softmax is the
#     draft distribution of the depth-k tokens, and all heads read the same
#     hidden state, so every depth-k node of a sequence shares it)
# --------------------------------------------------------------------------
def _softmax_rows(z: np.ndarray) -> np.ndarray:
    z = _f64(z)
    e = np.exp(z - z.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def accept_speculative_lm(x_t, w_lm, draft_logits, node_tokens, parents, uniforms,
                          D: int) -> Dict[str, np.ndarray]:
    """accept_speculative with P_t[b, r] = softmax(W_lm x_t[b, r]) (x_t [B, N+1, d], W_lm
    [V, d]) and P_d[b, r] = softmax(draft_logits[b, k]) where k = depth of the node of row r
    (0 for the prefix row; draft_logits [B, D, V], row k for the nodes at depth k+1).  Rows of
    nodes at depth D have no children; their draft row is never read (zeros here)."""
    x_t, w_lm, dl = _f64(x_t), _f64(w_lm), _f64(draft_logits)
    B, R, _ = x_t.shape
    N = R - 1
    p_t = _softmax_rows(x_t @ w_lm.T)
    depth = build_tree(parents)["depth"]
    p_d = np.zeros_like(p_t)
    for r in range(R):
        k = 0 if r == 0 else int(depth[r - 1])
        if k < D:
            p_d[:, r] = _softmax_rows(dl[:, k])
    return accept_speculative(p_t, p_d, node_tokens, parents, uniforms, D)


# --------------------------------------------------------------------------
# 7. Commit of the accepted path ("Multi-Token Prediction: Draft-Model-Free
#    Speculative Decoding", "The 2D Tree Attention Mask": the engine commits
#    the longest accepted path, and each node sees exactly its ancestors, so
#    the kept path continues the prefix causally; "Production Deployment
#    Guidelines": the KV entries of unselected branches are culled).
#    Reading: the tree's K/V rows sit after the prefix in node order; keeping
#    the path means moving its rows to the front of that block and growing the
#    prefix by its length.
# --------------------------------------------------------------------------
def kv_commit(k_cache, v_cache, prefix_len, path_nodes, accept_len, N: int):
    """New (k_cache, v_cache, prefix_len) after keeping each sequence's accepted path.

    k_cache/v_cache [B, Hkv, L_cap, dh]; row L_b + i holds tree node i.  For sequence b with
    len = accept_len[b] and path = path_nodes[b][:len], row L_b + j of the result is row
    L_b + path[j] of the input (every KV head), other rows are unchanged, and the prefix
    becomes L_b + len.  Raises ValueError for a path that is not a valid accepted path
    (len outside [0, D], a node outside [j, N), or L_b + N beyond L_cap)."""
    k_new, v_new = np.array(k_cache, copy=True), np.array(v_cache, copy=True)
    L_cap = k_new.shape[2]
    D = np.asarray(path_nodes).shape[1]
    prefix_new = np.array(prefix_len, dtype=np.int64, copy=True)
    for b in range(k_new.shape[0]):
        L, n = int(prefix_len[b]), int(accept_len[b])
        if L < 0 or L + N > L_cap or n < 0 or n > D:
            raise ValueError(f"sequence {b}: prefix {L} / length {n} out of range")
        for j in range(n):
            node = int(path_nodes[b][j])
            if node < j or node >= N:
                raise ValueError(f"sequence {b}: path node {node} at level {j}")
            k_new[b, :, L + j] = k_cache[b, :, L + node]
            v_new[b, :, L + j] = v_cache[b, :, L + node]
        prefix_new[b] = L + n
    return k_new, v_new, prefix_new


# --------------------------------------------------------------------------
# 8. Multi-candidate speculative acceptance ("Speculative Decoding & Medusa
#    Tree Attention", section 2, "The Acceptance Sampling Rule": accept x with
#    probability min(1, P_t(x)/P_d(x)), otherwise draw from
#    normalize(max(0, P_t - P_d)); "Multi-Token Prediction: Draft-Model-Free
#    Speculative Decoding", "The 2D Tree Attention Mask": the tree is evaluated
#    by rejection sampling and the longest accepted path is committed).
#    Reading for several candidates under one node: the siblings are tested in
#    index order, and after each rejection the residual distribution takes the
#    place of the target for the next sibling (the replacement draw of the
#    single-candidate rule is made from a further draft sample instead).  When
#    the candidates are independent draws from the parent row's P_d, every
#    emitted token follows P_t (the recursive form of the rule, published as
#    multi-step speculative sampling in SpecInfer).
# --------------------------------------------------------------------------
def accept_multicandidate(p_target, p_draft, node_tokens, parents, uniforms,
                          D: int) -> Dict[str, np.ndarray]:
    """Lossless acceptance over a candidate tree with several candidates per node.

    p_target/p_draft [B, N+1, V] (row 0 = after the prefix, row i+1 = after node i);
    uniforms [B, N+1] in [0, 1).  Starting at the prefix with P = P_t[row], the children
    of the current node are tested in index order: child i with token x has
    alpha_i = min(1, P(x) / P_d[row](x)) (1 when P_d(x) = 0) and is accepted iff
    u[b, i] < alpha_i; the walk then moves to it (P = P_t of its row).  After a rejection
    P = normalize(max(0, P - P_d[row])) (P_t[row] when that is all zero) and the next
    sibling is tested.  When a node has no children left, the extra token is drawn from
    the current P with u[b, N] by inverse CDF.  alpha is -1 for nodes never tested;
    node_accept marks the path."""
    p_t, p_d = _f64(p_target), _f64(p_draft)
    u = _f64(uniforms)
    B = p_t.shape[0]
    N = len(parents)
    kids: Dict[int, List[int]] = {}
    for i in range(N):
        kids.setdefault(int(parents[i]), []).append(i)
    alpha = np.full((B, N), -1.0)
    accepted = np.zeros((B, N), dtype=bool)
    res = []
    for b in range(B):
        node, path = -1, []
        P = p_t[b, 0]
        moved = True
        while moved:
            moved = False
            Q = p_d[b, node + 1]
            for c in kids.get(node, []):
                x = int(node_tokens[b, c])
                alpha[b, c] = 1.0 if Q[x] == 0.0 else min(1.0, P[x] / Q[x])
                if u[b, c] < alpha[b, c]:
                    accepted[b, c] = True
                    path.append(c)
                    node = c
                    P = p_t[b, c + 1]
                    moved = True
                    break
                r = np.maximum(0.0, P - Q)
                P = r / r.sum() if r.sum() > 0.0 else p_t[b, node + 1]
        tok = _inverse_cdf(P, u[b, N])
        res.append((path, [int(node_tokens[b, n]) for n in path], tok))
    acc_len, path_nodes, out_tokens = _pack(res, B, D)
    return {"accept_len": acc_len, "path_nodes": path_nodes, "out_tokens": out_tokens,
            "node_accept": accepted, "alpha": alpha}


# --------------------------------------------------------------------------
# 9. Dynamic (confidence-ranked) tree ("Multi-Token Prediction: Draft-Model-Free
#    Speculative Decoding", section "2. EAGLE & EAGLE-2: Feature-Level
#    Autoregression": the tree is shaped by the candidates' confidence, deeper
#    where the predictions are sure and wider where they are not; "Production
#    Deployment Guidelines", "Dynamic Tree Depth Tuning": depth and the number
#    of candidate paths are tuned per workload).  Reading: a node is a
#    path of candidate ranks (r_1 .. r_d), one per Medusa head, scored by the
#    log of its joint probability sum_k log p_k(r_k); the tree is the N
#    best-scoring paths.  A path never scores above its prefix, so the set is
#    a tree.  Ties: higher score first, then smaller depth, then smaller ranks
#    in order from the first head.  Nodes are laid out breadth first, children
#    of a node in rank order.
# --------------------------------------------------------------------------
def dynamic_tree(cand_ids, cand_vals, cand_lse, s_per_depth: Sequence[int],
                 N: int) -> Dict[str, object]:
    """The N most probable candidate paths of each sequence, as a tree.

    cand_ids / cand_vals [B, D, s_max]: head k's candidates, best first (ids and logits);
    cand_lse [B, D] (log-sum-exp of head k's logits) or None when cand_vals already hold
    log-probabilities; log-probabilities above 0 count as 0.  Only the first s_per_depth[k]
    candidates of head k are used.
    Returns per sequence lists: parents, depth (1-based), tokens, score (fp64 joint
    log-probability, summed from the first head on), ranks, and the ancestor sets."""
    ids = np.asarray(cand_ids)
    vals = _f64(cand_vals)
    B, D, _ = vals.shape
    # log-probabilities, clamped at 0 (a dominant token's val - lse can round above 0), so
    # that no path scores above its prefix
    logp = np.minimum(0.0, vals - (_f64(cand_lse)[:, :, None] if cand_lse is not None else 0.0))
    out = {"parents": [], "depth": [], "tokens": [], "score": [], "ranks": [], "anc": []}
    for b in range(B):
        paths = []
        stack = [((), 0.0)]
        while stack:
            ranks, sc = stack.pop()
            d = len(ranks)
            if d == D:
                continue
            for r in range(int(s_per_depth[d])):
                s2 = sc + logp[b, d, r]
                paths.append((ranks + (r,), s2))
                stack.append((ranks + (r,), s2))
        if len(paths) < N:
            raise ValueError("fewer candidate paths than tree nodes")
        paths.sort(key=lambda t: (-t[1], len(t[0]), t[0]))
        chosen = {rk: sc for rk, sc in paths[:N]}
        order = []                      # breadth first; children in rank order
        pos = {(): -1}
        for d in range(1, D + 1):
            level = [rk for rk in chosen if len(rk) == d]
            level.sort(key=lambda rk: (pos[rk[:-1]], rk[-1]))
            for rk in level:
                pos[rk] = len(order)
                order.append(rk)
        parents = [pos[rk[:-1]] for rk in order]
        out["parents"].append(parents)
        out["depth"].append([len(rk) for rk in order])
        out["tokens"].append([int(ids[b, len(rk) - 1, rk[-1]]) for rk in order])
        out["score"].append([chosen[rk] for rk in order])
        out["ranks"].append(order)
        out["anc"].append(build_tree(parents)["anc"])
    return out
