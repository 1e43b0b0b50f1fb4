"""GPU parity of the target LM head (mv_lm_head_argmax) and of greedy acceptance fed with its
argmax ids (mv_accept_paths with MV_TARGET_IDS), against the oracle."""
import numpy as np
import pytest
import torch

from oracle import medusa_oracle as O
from medusa_tree_attention_verify_amd import _lib as L
from medusa_tree_attention_verify_amd import ops
from medusa_tree_attention_verify_amd import workloads as W
from medusa_tree_attention_verify_amd.workloads import branching_tree
from tests.gpu_util import assert_fp32, dev, dev_i32, host, require_gpu

pytestmark = pytest.mark.gpu


def _inputs(T, d, V, seed):
    x = W.normal(seed, "lm_x", (T, d), 1.0, bf16=True)
    w = W.normal(seed, "lm_w", (V, d), 1.0 / np.sqrt(d), bf16=True)
    return x, w


def _check_ids(got, z, rows=None):
    """Greedy ids exact, except where the oracle's top two logits are within 1e-4 relative
    (both are then accepted and counted)."""
    rows = range(z.shape[0]) if rows is None else rows
    ties = 0
    for i, t in enumerate(rows):
        zr = z[i]
        top = zr.max()
        want = int(np.flatnonzero(zr == top)[0])
        if int(got[t]) != want:
            assert zr[int(got[t])] >= top - 1e-4 * max(1.0, abs(top)), (t, int(got[t]), want)
            ties += 1
    return ties


@pytest.mark.parametrize("T,d,V", [(1, 256, 1000), (5, 256, 999), (33, 512, 777),
                                   (128, 256, 1500), (65, 1024, 5000),
                                   (17, 96, 500), (40, 192, 777),   # 3 and 6 k-steps: batches of 1 and 2
                                   # from 129 rows the tiled kernel (128 target rows per tile; 256 from
                                   # 2049): ragged target and vocabulary tiles, 2 and 6 stages of d
                                   (129, 512, 999), (130, 256, 1500), (300, 256, 1500),
                                   (2100, 128, 300), (1100, 256, 999), (200, 384, 2000),
                                   (150, 160, 500)])   # d % 128 != 0: streaming kernel in groups of 128
def test_lm_head_small_shapes(T, d, V):
    require_gpu()
    print(f"lm head T={T} d={d} V={V}", flush=True)
    x, w = _inputs(T, d, V, T + V)
    got = ops.lm_head_argmax(dev(x, torch.bfloat16), dev(w, torch.bfloat16))
    torch.cuda.synchronize()
    ref = O.lm_head_argmax(x, w)
    assert _check_ids(host(got["ids"]), ref["logits"]) == 0
    assert_fp32(host(got["max"]), ref["max"], atol=1e-4, what="max logit")
    assert_fp32(host(got["lse"]), ref["lse"], atol=1e-4, what="lse")


def test_lm_head_llama8b_shape():
    """The verify rows of the Llama-3-8B-shaped step: T = 65 (prefix row + 64 nodes), d = 4096,
    V = 32000; every row compared."""
    require_gpu()
    x, w = _inputs(65, 4096, 32000, 8)
    got = ops.lm_head_argmax(dev(x, torch.bfloat16), dev(w, torch.bfloat16))
    torch.cuda.synchronize()
    ref = O.lm_head_argmax(x, w)
    ties = _check_ids(host(got["ids"]), ref["logits"])
    print("near-tie rows:", ties)
    assert ties <= 1
    assert_fp32(host(got["max"]), ref["max"], atol=1e-3, what="max logit")
    assert_fp32(host(got["lse"]), ref["lse"], atol=1e-3, what="lse")


@pytest.mark.parametrize("B,d,V", [(8, 4096, 32000), (8, 8192, 32000), (64, 4096, 32000),
                                   (64, 4096, 128256)])
def test_lm_head_batched_verify_rows_sampled(B, d, V):
    """A batch of verify steps (B x 65 rows: T = 520 takes the tiled kernel with 128-row target
    tiles, T = 4160 with 256-row tiles), up to the 64-sequence serving batch over the Llama-3
    vocabulary and the 70B share's d = 8192: the GPU computes every row, the oracle recomputes
    16 sampled rows spread over the tiles, including tile edges and the last (ragged) tile."""
    require_gpu()
    T = B * 65
    print(f"lm head batched T={T} d={d} V={V}", flush=True)
    x, w = _inputs(T, d, V, 10 + B + d + V)
    got = ops.lm_head_argmax(dev(x, torch.bfloat16), dev(w, torch.bfloat16))
    torch.cuda.synchronize()
    rng = np.random.default_rng(B)
    rows = sorted(set([0, 127, 128, 255, 256, T - 1] + rng.choice(T, 10, replace=False).tolist()))
    ref = O.lm_head_argmax(x[rows], w)
    ids, mx, lse = host(got["ids"]), host(got["max"]), host(got["lse"])
    assert _check_ids(ids, ref["logits"], rows) <= 1
    assert_fp32(mx[rows], ref["max"], atol=1e-3, what="max logit")
    assert_fp32(lse[rows], ref["lse"], atol=1e-3, what="lse")


def test_lm_head_full_vocab_sampled():
    """V = 128256 (the Llama-3 vocabulary), T = 65, d = 4096: the GPU computes every row, the
    oracle recomputes 8 sampled rows."""
    require_gpu()
    x, w = _inputs(65, 4096, 128256, 9)
    got = ops.lm_head_argmax(dev(x, torch.bfloat16), dev(w, torch.bfloat16))
    torch.cuda.synchronize()
    rows = [0, 7, 19, 31, 40, 52, 60, 64]
    ref = O.lm_head_argmax(x[rows], w)
    ids, mx, lse = host(got["ids"]), host(got["max"]), host(got["lse"])
    assert _check_ids(ids, ref["logits"], rows) <= 1
    assert_fp32(mx[rows], ref["max"], atol=1e-3, what="max logit")
    assert_fp32(lse[rows], ref["lse"], atol=1e-3, what="lse")


def test_greedy_acceptance_from_lm_head_ids():
    """A 64-node (4,3,2,1) tree, 3 sequences: the LM head's argmax ids drive greedy acceptance
    (no [B, N+1, V] logits on the GPU); the oracle accepts on its own fp64 logits.  Tree tokens
    follow the oracle's greedy token of the parent row with probability 0.7."""
    require_gpu()
    parents = branching_tree((4, 3, 2, 1))
    N, B, d, V = len(parents), 3, 256, 1000
    D = int(O.build_tree(parents)["depth"].max())
    x, w = _inputs(B * (N + 1), d, V, 21)
    ref_lm = O.lm_head_argmax(x, w)
    g = ref_lm["ids"].reshape(B, N + 1)
    rng = W.rng_for(21, "lm_tokens")
    toks = np.empty((B, N), dtype=np.int32)
    for b in range(B):
        for i, p in enumerate(parents):
            toks[b, i] = g[b, p + 1] if rng.random() < 0.7 else rng.integers(0, V)
    got_lm = ops.lm_head_argmax(dev(x, torch.bfloat16), dev(w, torch.bfloat16))
    ids = got_lm["ids"].view(B, N + 1)
    got = ops.accept_paths(L.MV_ACCEPT_GREEDY, dev_i32(parents), dev_i32(toks), ids, D, vocab=V)
    torch.cuda.synchronize()
    assert _check_ids(host(got_lm["ids"]), ref_lm["logits"]) == 0
    ref = O.accept_greedy(ref_lm["logits"].reshape(B, N + 1, V), toks, parents, D)
    for k in ("accept_len", "path_nodes", "out_tokens"):
        np.testing.assert_array_equal(host(got[k]), ref[k], err_msg=k)
    np.testing.assert_array_equal(host(got["node_accept"]).astype(bool), ref["node_accept"])
    print("accept lengths", host(got["accept_len"]).tolist())
