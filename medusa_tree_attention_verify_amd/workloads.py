"""Seeded synthetic workloads for Medusa tree verification.

This module only *draws inputs*. It holds none of the verification
arithmetic (no head GEMVs, no tree masks, no attention, no acceptance rule);
both the HIP path and the CPU oracle consume what it returns.

Conventions
-----------
* Every draw comes from NumPy's PCG64.  Large tensors are filled in fixed
  blocks of ``_BLOCK`` elements, each block from its own child of a
  ``SeedSequence`` keyed by (seed, tensor name), so the values do not depend
  on how many threads fill them.
* ``N(0, s)`` means mean 0 and *standard deviation* s.
* bf16 tensors are returned as float32 arrays whose values are exactly
  representable in bf16 (round-to-nearest-even applied once here);
  :func:`bf16_bits` gives the raw 16-bit patterns to upload.
* Trees are parent arrays in topological (BFS-by-depth) order; parent -1
  means "child of the last prefix token".

The five named workloads follow the configurations the method is measured
on: a tiny fp32 case, a Llama-3-8B-shaped layer, a 70B-shaped one-GPU share
at batch 8, a 131072-token context with a 212-node tree, and a batch-64
speculative-sampling case.
"""
from __future__ import annotations

import dataclasses
import hashlib
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

_BLOCK = 1 << 22


# --------------------------------------------------------------------------
# trees
# --------------------------------------------------------------------------
def branching_tree(widths: Sequence[int]) -> List[int]:
    """Parent array of a full tree: every node at depth k has widths[k] children.

    Nodes are numbered breadth first, so the depth-1 nodes come first (their
    parent is -1), then all depth-2 nodes grouped by parent, and so on.
    """
    parents: List[int] = []
    level = [-1]
    for w in widths:
        nxt = []
        for p in level:
            for _ in range(w):
                parents.append(p)
                nxt.append(len(parents) - 1)
        level = nxt
    return parents


def chain_tree(depth: int) -> List[int]:
    return [-1] + list(range(depth - 1))


def two_chains_tree() -> List[int]:
    """Two depth-4 chains hanging off the top-2 depth-1 candidates (8 nodes)."""
    return [-1, -1, 0, 1, 2, 3, 4, 5]


# --------------------------------------------------------------------------
# workload descriptions
# --------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    dtype: str                       # "f32" or "bf16" (attention, heads, greedy logits)
    B: int
    Hq: int
    Hkv: int
    dh: int
    parents: Tuple[int, ...]
    prefix: Tuple[int, int]          # L_b ~ U{lo..hi} (inclusive); lo == hi -> fixed
    depth_widths: Tuple[int, ...]    # s_k: candidates per depth (tree depth = len)
    # Medusa heads (K == 0 -> heads are not part of the step)
    d: int = 0
    V: int = 0
    K: int = 0
    head_widths: Tuple[int, ...] = ()
    lm_width: int = 0                # depth-1 candidates taken from the target's own row 0
    weight_std: float = 0.0          # 0 -> N(0,1)/sqrt(fan_in)
    # acceptance
    accept: str = "greedy"           # "greedy", "speculative", "multicand" or "none"
    accept_V: int = 0
    target_std: float = 2.0
    plant_p: float = 0.0             # probability that a parent row's argmax is one of its children
    draft_noise_std: float = 1.0
    dynamic_nodes: int = 0           # > 0: per-sequence tree of the N most probable head paths
    draft_tokens: str = "top"        # sampling modes: children's tokens are the draft row's
                                     # top tokens ("top") or independent draws from it ("sampled")
    qkv_scaled: bool = False         # Q,K,V divided by sqrt(dh)
    target_head: bool = False        # greedy target from the LM head: W_lm [accept_V, d] times
                                     # the verify rows' hidden states x_t [B, N+1, d]

    @property
    def N(self) -> int:
        return len(self.parents)

    @property
    def D(self) -> int:
        return len(self.depth_widths)

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def has_heads(self) -> bool:
        return self.K > 0

    def scaled(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


_T4321 = tuple(branching_tree((4, 3, 2, 1)))
_T4442 = tuple(branching_tree((4, 4, 4, 2)))

WORKLOADS: Dict[str, Workload] = {
    # tiny fp32, batch 1
    "c1": Workload(name="tiny-fp32", dtype="f32", B=1, Hq=4, Hkv=4, dh=64,
                   parents=tuple(two_chains_tree()), prefix=(128, 128),
                   depth_widths=(2, 1, 1, 1), d=256, V=1000, K=3,
                   head_widths=(1, 1, 1), lm_width=2, weight_std=0.0,
                   accept="greedy", accept_V=1000, target_std=2.0,
                   plant_p=0.0, qkv_scaled=True),
    # Llama-3-8B-shaped layer, bf16, batch 1
    "c2": Workload(name="llama3-8b-layer", dtype="bf16", B=1, Hq=32, Hkv=8, dh=128,
                   parents=_T4321, prefix=(4096, 4096), depth_widths=(4, 3, 2, 1),
                   d=4096, V=32000, K=4, head_widths=(4, 3, 2, 1), weight_std=0.02,
                   accept="greedy", accept_V=32000, target_std=2.0, plant_p=0.6),
    # 70B-shaped one-GPU share, bf16, batch 8
    "c3": Workload(name="70b-share-b8", dtype="bf16", B=8, Hq=64, Hkv=8, dh=128,
                   parents=_T4321, prefix=(8192, 32768), depth_widths=(4, 3, 2, 1),
                   d=8192, V=32000, K=4, head_widths=(4, 3, 2, 1), weight_std=0.02,
                   accept="greedy", accept_V=32000, target_std=2.0, plant_p=0.6),
    # long context, attention only
    "c4": Workload(name="long-ctx-131k", dtype="bf16", B=1, Hq=64, Hkv=8, dh=128,
                   parents=_T4442, prefix=(131072, 131072), depth_widths=(4, 4, 4, 2),
                   accept="none"),
    # batched stochastic serving
    "c5": Workload(name="spec-serving-b64", dtype="bf16", B=64, Hq=32, Hkv=8, dh=128,
                   parents=_T4321, prefix=(512, 8192), depth_widths=(4, 3, 2, 1),
                   accept="speculative", accept_V=128256, target_std=3.0,
                   draft_noise_std=1.0),
    # batched serving with several independent draft samples per node and the
    # sibling-recursive (lossless) acceptance rule
    "c7": Workload(name="spec-serving-b64-multicand", dtype="bf16", B=64, Hq=32, Hkv=8, dh=128,
                   parents=_T4321, prefix=(512, 8192), depth_widths=(4, 3, 2, 1),
                   accept="multicand", accept_V=128256, target_std=3.0,
                   draft_noise_std=1.0, draft_tokens="sampled"),
    # the Llama-3-8B-shaped step with a dynamic tree: each head proposes 10 candidates and the
    # tree is the 64 most probable paths (parents below only fix N = 64 for the shapes)
    "c8": Workload(name="llama3-8b-layer-dyntree", dtype="bf16", B=1, Hq=32, Hkv=8, dh=128,
                   parents=_T4321, prefix=(4096, 4096), depth_widths=(10, 10, 10, 10),
                   d=4096, V=32000, K=4, head_widths=(10, 10, 10, 10), weight_std=0.02,
                   accept="greedy", accept_V=32000, target_std=2.0, plant_p=0.6,
                   dynamic_nodes=64),
    "c6": Workload(name="llama3-8b-layer-lmhead", dtype="bf16", B=1, Hq=32, Hkv=8, dh=128,
                   parents=_T4321, prefix=(4096, 4096), depth_widths=(4, 3, 2, 1),
                   d=4096, V=32000, K=4, head_widths=(4, 3, 2, 1), weight_std=0.02,
                   accept="greedy", accept_V=32000, plant_p=0.6, target_head=True),
    # the same step with speculative acceptance: the target from the LM head, the draft of
    # depth k from Medusa head k's logits, seeded uniforms
    "c9": Workload(name="llama3-8b-layer-lmhead-spec", dtype="bf16", B=1, Hq=32, Hkv=8, dh=128,
                   parents=_T4321, prefix=(4096, 4096), depth_widths=(4, 3, 2, 1),
                   d=4096, V=32000, K=4, head_widths=(4, 3, 2, 1), weight_std=0.02,
                   accept="speculative", accept_V=32000, target_head=True),
    # the batched serving step driven by the target LM head: 64 sequences x 65 verify rows
    # through W_lm [128256, 4096]; the draft of depth k is a separate draft's logits row
    # [B, D, V] (no Medusa heads at this batch), whose top candidates also build the tree
    "c10": Workload(name="spec-serving-b64-lmhead", dtype="bf16", B=64, Hq=32, Hkv=8, dh=128,
                    parents=_T4321, prefix=(512, 8192), depth_widths=(4, 3, 2, 1), d=4096,
                    accept="speculative", accept_V=128256, target_head=True),
}


# --------------------------------------------------------------------------
# seeded block generation
# --------------------------------------------------------------------------
def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _seed_for(seed: int, name: str) -> np.random.SeedSequence:
    h = int.from_bytes(hashlib.sha256(name.encode()).digest()[:8], "little")
    return np.random.SeedSequence([int(seed), h])


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); returns float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) & np.uint32(0xFFFF0000)
    return r.view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Raw bf16 bit patterns of float32 values that are already bf16-exact."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    return (x.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def normal(seed: int, name: str, shape, std: float = 1.0, bf16: bool = False) -> np.ndarray:
    """N(0, std) float32 draws (optionally rounded to bf16), block-seeded."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32)
    nb = (n + _BLOCK - 1) // _BLOCK
    kids = _seed_for(seed, name).spawn(max(nb, 1))

    def fill(i):
        sl = out[i * _BLOCK:(i + 1) * _BLOCK]
        g = np.random.Generator(np.random.PCG64(kids[i]))
        g.standard_normal(out=sl, dtype=np.float32)
        if std != 1.0:
            sl *= np.float32(std)
        if bf16:
            sl[:] = round_bf16(sl)

    if nb <= 1:
        for i in range(nb):
            fill(i)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(nb)))
    return out.reshape(shape)


def rng_for(seed: int, name: str) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(_seed_for(seed, name)))


def children_of(parents: Sequence[int]) -> Dict[int, List[int]]:
    """Map parent index (-1 = prefix) to its children in index order."""
    ch: Dict[int, List[int]] = {}
    for i, p in enumerate(parents):
        ch.setdefault(int(p), []).append(i)
    return ch


# --------------------------------------------------------------------------
# per-part inputs
# --------------------------------------------------------------------------
def gen_prefix_lens(w: Workload, seed: int) -> np.ndarray:
    lo, hi = w.prefix
    if lo == hi:
        return np.full(w.B, lo, dtype=np.int32)
    return rng_for(seed, "prefix_len").integers(lo, hi, size=w.B, endpoint=True).astype(np.int32)


def gen_heads(w: Workload, seed: int) -> Dict[str, np.ndarray]:
    """h [B,d], W_res [K,d,d] (out,in), W_head [K,V,d]."""
    bf = w.dtype == "bf16"
    if w.weight_std > 0:
        h = normal(seed, "h", (w.B, w.d), 1.0, bf)
        w_res = normal(seed, "w_res", (w.K, w.d, w.d), w.weight_std, bf)
        w_head = normal(seed, "w_head", (w.K, w.V, w.d), w.weight_std, bf)
    else:
        s = 1.0 / np.sqrt(w.d)
        h = normal(seed, "h", (w.B, w.d), s, bf)
        w_res = normal(seed, "w_res", (w.K, w.d, w.d), s, bf)
        w_head = normal(seed, "w_head", (w.K, w.V, w.d), s, bf)
    return {"h": h, "w_res": w_res, "w_head": w_head}


def gen_attention(w: Workload, seed: int, prefix_len: Optional[np.ndarray] = None) -> Dict[str, np.ndarray]:
    """Q [B,N,Hq,dh]; K/V cache [B,Hkv,L_cap,dh] with the tree's K/V at rows [L_b, L_b+N)."""
    bf = w.dtype == "bf16"
    if prefix_len is None:
        prefix_len = gen_prefix_lens(w, seed)
    L_cap = int(prefix_len.max()) + w.N
    s = 1.0 / np.sqrt(w.dh) if w.qkv_scaled else 1.0
    q = normal(seed, "q", (w.B, w.N, w.Hq, w.dh), s, bf)
    k = normal(seed, "k_cache", (w.B, w.Hkv, L_cap, w.dh), s, bf)
    v = normal(seed, "v_cache", (w.B, w.Hkv, L_cap, w.dh), s, bf)
    return {"q": q, "k_cache": k, "v_cache": v, "prefix_len": prefix_len.astype(np.int32),
            "L_cap": L_cap}


def gen_target_head(w: Workload, seed: int) -> Dict[str, np.ndarray]:
    """Hidden states of the verify rows x_t [B, N+1, d] ~ N(0,1) and the LM-head weight
    W_lm [accept_V, d] ~ N(0, 1/d) (rows of norm ~1), both rounded to bf16."""
    return {"x_t": normal(seed, "x_t", (w.B, w.N + 1, w.d), 1.0, True),
            "w_lm": normal(seed, "w_lm", (w.accept_V, w.d), 1.0 / np.sqrt(w.d), True)}


def gen_draft_logits(w: Workload, seed: int) -> np.ndarray:
    """A draft's logits for depths 1..D of every sequence, [B, D, accept_V] ~ N(0, 1) rounded
    to bf16 (the draft distribution of depth k is the softmax of row k)."""
    return normal(seed, "draft_logits", (w.B, w.D, w.accept_V), 1.0, True)


def gen_uniforms(w: Workload, seed: int) -> np.ndarray:
    """Uniforms [B, N+1] in [0, 1) for a speculative step (float32)."""
    return rng_for(seed, "uniforms").random((w.B, w.N + 1), dtype=np.float32)


def plant_target_head(x_t: np.ndarray, w_lm: np.ndarray, parents: Sequence[int],
                      node_tokens: np.ndarray, seed: int, p: float) -> np.ndarray:
    """Make each parent row's greedy token one of its children with probability p, through the
    hidden state: the row becomes 8 x the chosen token's W_lm row (rounded to bf16), whose
    logit (~8) then clears every other one (~N(0, (8/sqrt(d))^2)).  Other rows keep their
    random state.  Works in place and returns x_t."""
    rng = rng_for(seed, "plant_lm")
    ch = children_of(parents)
    for b in range(x_t.shape[0]):
        for par in sorted(ch):
            if rng.random() < p:
                kids = ch[par]
                t = int(node_tokens[b, kids[int(rng.integers(len(kids)))]])
                x_t[b, par + 1] = round_bf16(np.float32(8.0) * w_lm[t])
    return x_t


def gen_target_logits(w: Workload, seed: int) -> np.ndarray:
    """Target logits [B, N+1, V] ~ N(0, target_std) (float32, not yet rounded)."""
    return normal(seed, "target_logits", (w.B, w.N + 1, w.accept_V), w.target_std, False)


def plant_greedy(logits: np.ndarray, parents: Sequence[int], node_tokens: np.ndarray,
                 seed: int, p: float) -> np.ndarray:
    """Make each parent row's greedy choice one of its children with probability p.

    Row 0 is the prefix end; row i+1 belongs to node i.  For every row that has
    children: with probability p one child (uniform) gets its token's logit set
    to the row maximum + 1 (a unique maximum); otherwise every child token's
    logit is pushed below the row minimum so that no child can match.
    Works in place on a float32 array and returns it.
    """
    rng = rng_for(seed, "plant")
    ch = children_of(parents)
    B = logits.shape[0]
    for b in range(B):
        for par in sorted(ch):
            row = logits[b, par + 1]
            kids = ch[par]
            toks = [int(node_tokens[b, c]) for c in kids]
            if rng.random() < p:
                t = toks[int(rng.integers(len(toks)))]
                row[t] = row.max() + np.float32(1.0)
            else:
                lo = row.min() - np.float32(1.0)
                for t in toks:
                    row[t] = lo
    return logits


def gen_speculative(w: Workload, seed: int, rows: Optional[Sequence[int]] = None) -> Dict[str, np.ndarray]:
    """P_target, P_draft [B, N+1, V] float32 probabilities, uniforms [B, N+1], node tokens [B, N].

    P_target = softmax(N(0, target_std) logits); P_draft = softmax(the same logits
    + N(0, draft_noise_std) noise).  Children of a row get, in index order, the
    draft's highest-probability tokens of that row (the draft's own proposals), or with
    ``draft_tokens == "sampled"`` independent draws from that row (repeats allowed).
    ``rows`` restricts generation to a subset of sequences (others are left 0).
    """
    B, R, V = w.B, w.N + 1, w.accept_V
    p_t = np.zeros((B, R, V), dtype=np.float32)
    p_d = np.zeros((B, R, V), dtype=np.float32)
    kids = _seed_for(seed, "spec_rows").spawn(B)
    rows = list(range(B)) if rows is None else list(rows)

    def seq(b):
        g = np.random.Generator(np.random.PCG64(kids[b]))
        lt = g.standard_normal((R, V), dtype=np.float32).astype(np.float64) * w.target_std
        ld = lt + g.standard_normal((R, V), dtype=np.float32).astype(np.float64) * w.draft_noise_std
        for src, dst in ((lt, p_t), (ld, p_d)):
            e = np.exp(src - src.max(axis=1, keepdims=True))
            dst[b] = (e / e.sum(axis=1, keepdims=True)).astype(np.float32)

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(seq, rows))
    ch = children_of(w.parents)
    node_tokens = np.zeros((B, w.N), dtype=np.int32)
    if w.draft_tokens == "sampled":
        g = rng_for(seed, "draft_draws")
        for b in rows:
            for par, kids_ in ch.items():
                cdf = np.cumsum(p_d[b, par + 1].astype(np.float64))
                u = g.random(len(kids_)) * cdf[-1]
                node_tokens[b, kids_] = np.minimum(np.searchsorted(cdf, u, side="right"), V - 1)
        uniforms = rng_for(seed, "uniforms").random((B, R), dtype=np.float32)
        return {"p_target": p_t, "p_draft": p_d, "node_tokens": node_tokens, "uniforms": uniforms}
    for b in rows:
        for par, kids_ in ch.items():
            row = p_d[b, par + 1]
            c = len(kids_)
            top = np.argpartition(-row, c - 1)[:c] if c < V else np.arange(V)
            order = sorted(top.tolist(), key=lambda j: (-row[j], j))
            for c, t in zip(kids_, order):
                node_tokens[b, c] = int(t)
    uniforms = rng_for(seed, "uniforms").random((B, R), dtype=np.float32)
    return {"p_target": p_t, "p_draft": p_d, "node_tokens": node_tokens, "uniforms": uniforms}
