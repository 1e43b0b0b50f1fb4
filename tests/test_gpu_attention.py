"""GPU parity of tree-masked GQA attention against the oracle: mv_tree_attn_verify and the
launch mv_tree_attn_verify_beside (persistent workgroups on half of the CUs), on the same cases."""
import numpy as np
import pytest
import torch

from oracle import medusa_oracle as O
from medusa_tree_attention_verify_amd import _lib as L
from medusa_tree_attention_verify_amd import ops
from medusa_tree_attention_verify_amd import workloads as W
from medusa_tree_attention_verify_amd.workloads import branching_tree, chain_tree
from tests.gpu_util import assert_bf16, assert_fp32, dev, dev_i32, host, require_gpu

pytestmark = pytest.mark.gpu


def _run(wl, seed, lens=None, select=None, beside=False):
    print(f"attn {wl.name} B={wl.B} N={wl.N} Hq={wl.Hq} Hkv={wl.Hkv} dh={wl.dh} "
          f"prefix={wl.prefix} lens={lens} seed={seed} beside={beside}", flush=True)
    x = W.gen_attention(wl, seed, None if lens is None else np.asarray(lens, np.int32))
    dt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    tree = O.build_tree(list(wl.parents))
    parents = dev_i32(wl.parents)
    anc = ops.build_tree_mask(parents)["anc_mask"]
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    max_L = int(x["prefix_len"].max())
    q = dev(x["q"], dt)
    # outputs start as NaN, so a row the kernels never write is caught below
    out0 = torch.full_like(q, float("nan"))
    lse0 = torch.full((wl.B, wl.Hq, wl.N), float("nan"), dtype=torch.float32, device="cuda")
    out, lse = ops.tree_attn_verify(q, dev(x["k_cache"], dt), dev(x["v_cache"], dt),
                                    dev_i32(x["prefix_len"]), anc, max_L, status=status,
                                    out=out0, lse=lse0, beside=beside)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    assert bool(torch.isfinite(out).all()), "an output row was not written"
    assert bool(torch.isfinite(lse).all()), "an LSE entry was not written"
    ref = O.tree_attention(x["q"], x["k_cache"], x["v_cache"], x["prefix_len"], tree["anc"],
                           select=select)
    got_o, got_l = host(out), host(lse)
    if select is not None:
        idx = tuple(np.array(select).T)          # (b, h, i)
        b, h, i = idx
        go, ro = got_o[b, i, h], ref["out"][b, i, h]
        gl, rl = got_l[b, h, i], ref["lse"][b, h, i]
    else:
        go, ro, gl, rl = got_o, ref["out"], got_l, ref["lse"]
    if wl.dtype == "f32":
        assert_fp32(go, ro, what="out")
        assert_fp32(gl, rl, what="lse")
    else:
        assert_bf16(go, ro, what="out")
        assert_fp32(gl, rl, atol=1e-3, what="lse")


BESIDE = pytest.mark.parametrize("beside", [False, True], ids=["alone", "beside"])


@BESIDE
def test_attention_tiny_fp32(beside):
    require_gpu()
    _run(W.WORKLOADS["c1"], 1, beside=beside)


def _bf16(parents, B, Hq, Hkv, dh, L):
    return W.Workload(name="bf16-case", dtype="bf16", B=B, Hq=Hq, Hkv=Hkv, dh=dh,
                      parents=tuple(parents), prefix=(L, L), depth_widths=(1,))


@pytest.mark.parametrize("parents,B,Hq,Hkv,dh,lens", [
    ([-1], 2, 8, 2, 128, [37, 300]),                        # one node: plain decode
    (chain_tree(9), 1, 4, 1, 64, [20]),                     # chain: causal
    (branching_tree((4, 3, 2, 1)), 1, 32, 8, 128, [0]),     # empty prefix
    (branching_tree((4, 3, 2, 1)), 2, 32, 8, 128, [5, 130]),
    (branching_tree((4, 3, 2, 1)), 3, 16, 8, 64, [1, 511, 1000]),
    (branching_tree((2, 2)), 2, 8, 8, 128, [33, 64]),       # G = 1
    (branching_tree((4, 4, 4, 2)), 1, 16, 2, 128, [77]),    # 212 nodes, 7 mask words
    ([-1, 0, 1, 1, 0, -1, 5], 1, 8, 1, 64, [3]),            # forest (two roots)
])
@BESIDE
def test_attention_bf16_shapes(parents, B, Hq, Hkv, dh, lens, beside):
    require_gpu()
    wl = _bf16(parents, B, Hq, Hkv, dh, max(lens))
    _run(wl, 21, lens, beside=beside)


def _f32(parents, B, Hq, Hkv, dh, L):
    return W.Workload(name="f32-case", dtype="f32", B=B, Hq=Hq, Hkv=Hkv, dh=dh,
                      parents=tuple(parents), prefix=(L, L), depth_widths=(1,))


@pytest.mark.parametrize("parents,B,Hq,Hkv,dh,lens", [
    ([-1], 2, 8, 2, 128, [37, 300]),                        # one node, several chunks of keys
    (chain_tree(9), 1, 4, 1, 64, [20]),
    (branching_tree((4, 3, 2, 1)), 1, 8, 2, 128, [0]),      # empty prefix: exactly 64 keys
    (branching_tree((2, 2)), 2, 8, 8, 64, [59, 60]),        # 65 and 66 keys: one-key tail chunk
    (branching_tree((4, 4, 4, 2)), 1, 4, 2, 128, [77]),     # 212 nodes, 7 mask words
    ([-1, 0, 1, 1, 0, -1, 5], 3, 8, 4, 64, [3, 64, 129]),   # forest (two roots), ragged batch
])
def test_attention_fp32_shapes(parents, B, Hq, Hkv, dh, lens):
    """The fp32 path (one wave per query row, P.V in batches of V rows) at both head sizes,
    across chunk boundaries of its 64-key loop."""
    require_gpu()
    wl = _f32(parents, B, Hq, Hkv, dh, max(lens))
    _run(wl, 23, lens)


def _random_forest(n, seed):
    """Parent array of n nodes in topological order, roots (-1) allowed anywhere."""
    rng = np.random.default_rng(seed)
    return [-1] + [int(rng.integers(-1, i)) for i in range(1, n)]


@BESIDE
def test_attention_max_nodes(beside):
    """256 nodes (the largest tree: 8 mask words, 4 tree tiles), a random forest, G = 4."""
    require_gpu()
    wl = _bf16(_random_forest(256, 7), 2, 8, 2, 64, 700)
    _run(wl, 23, [100, 700], beside=beside)


@BESIDE
def test_attention_multichunk_with_empty_prefix(beside):
    """A split batch in which one sequence has no prefix (its rows skip the combine)."""
    require_gpu()
    wl = _bf16(branching_tree((4, 3, 2, 1)), 3, 32, 8, 128, 5000)
    _run(wl, 24, [0, 5000, 2049], beside=beside)


@BESIDE
def test_attention_multichunk_ragged(beside):
    """Prefixes long enough to be split into several chunks, ragged across the batch."""
    require_gpu()
    wl = _bf16(branching_tree((4, 3, 2, 1)), 4, 32, 8, 128, 6000)
    _run(wl, 22, [6000, 257, 4096, 1], beside=beside)


def test_attention_beside_more_indices_than_cus():
    """The persistent launch with far more workgroup indices than CUs (one sequence split
    into many chunks, 8 KV heads, 4 query tiles each) and with fewer (one short sequence):
    every row written, every row against the oracle."""
    require_gpu()
    wl = _bf16(branching_tree((4, 4, 4, 2)), 1, 32, 8, 64, 20000)
    rng = np.random.default_rng(27)
    sel = [(0, int(rng.integers(wl.Hq)), int(rng.integers(wl.N))) for _ in range(40)]
    sel += [(0, 0, 0), (0, wl.Hq - 1, wl.N - 1)]
    _run(wl, 28, [20000], select=sel, beside=True)
    _run(_bf16(branching_tree((2, 2)), 1, 4, 4, 128, 10), 29, [10], beside=True)


@BESIDE
def test_attention_balanced_split_two_query_tiles(beside):
    """A split batch with two query tiles per KV head (64/8 heads, 64 nodes) and very uneven
    prefixes (0 to 12000 keys), so the chunk plan is built on the device from the actual
    lengths: every output row must be written, sampled rows of every sequence (the first and
    the deepest node among them) match the oracle."""
    require_gpu()
    wl = _bf16(branching_tree((4, 3, 2, 1)), 6, 64, 8, 128, 12000)
    rng = np.random.default_rng(26)
    sel = []
    for b in range(wl.B):
        sel += [(b, int(rng.integers(wl.Hq)), int(rng.integers(wl.N))) for _ in range(4)]
        sel += [(b, int(rng.integers(wl.Hq)), 0), (b, int(rng.integers(wl.Hq)), wl.N - 1)]
    _run(wl, 25, [0, 1, 65, 3000, 9000, 12000], select=sel, beside=beside)


@BESIDE
def test_attention_llama8b_full(beside):
    """B=1, 32/8 heads, dh 128, prefix 4096, (4,3,2,1) tree: every output row."""
    require_gpu()
    _run(W.WORKLOADS["c2"], 2, beside=beside)


def test_attention_long_context_sampled():
    """Prefix 131072, 64/8 heads, 212-node tree: sampled rows incl. the deepest nodes."""
    require_gpu()
    wl = W.WORKLOADS["c4"]
    rng = np.random.default_rng(4)
    sel = [(0, int(rng.integers(64)), int(i)) for i in rng.integers(0, wl.N, size=24)]
    sel += [(0, 63, wl.N - 1), (0, 0, 0), (0, 7, 84), (0, 8, 211)]
    _run(wl, 4, select=sel)


@BESIDE
def test_attention_70b_share_sampled(beside):
    """Batch 8, 64/8 heads, prefixes drawn in [8192, 32768]: sampled rows of every sequence."""
    require_gpu()
    wl = W.WORKLOADS["c3"]
    rng = np.random.default_rng(3)
    sel = [(b, int(rng.integers(64)), int(rng.integers(64))) for b in range(8) for _ in range(3)]
    _run(wl, 3, select=sel, beside=beside)


@BESIDE
def test_attention_serving_b64_full_shape(beside):
    """The spec-serving attention shape at full size: batch 64, 32/8 heads, dh 128, the 64-node
    (4,3,2,1) tree, prefixes drawn in [512, 8192], with several equal lengths (the length
    ordering's tie rule), one empty prefix and one at the maximum.  Every output row must be
    written (NaN-filled beforehand); sampled rows of every one of the 64 sequences are compared
    with the oracle, including the first and the deepest node."""
    require_gpu()
    wl = W.WORKLOADS["c5"]
    lens = W.gen_prefix_lens(wl, 5).copy()
    lens[[3, 10, 20]] = lens[3]           # a three-way tie
    lens[[40, 41]] = 4096                 # a two-way tie, adjacent
    lens[[7, 50]] = lens[50]              # a tie far apart
    lens[63] = 0                          # no prefix: the tree alone
    lens[5] = 8192                        # the longest possible prefix
    rng = np.random.default_rng(55)
    sel = []
    for b in range(wl.B):
        sel += [(b, int(rng.integers(wl.Hq)), int(rng.integers(wl.N))) for _ in range(4)]
        sel += [(b, int(rng.integers(wl.Hq)), 0), (b, int(rng.integers(wl.Hq)), wl.N - 1)]
    _run(wl, 5, lens.tolist(), select=sel, beside=beside)


@pytest.mark.parametrize("B,lens,boost_rows", [
    (1, [3000], (2000, 2010)),        # one chunk: the jump comes after 31 ordinary tiles
    (2, [9000, 300], (8990, 9000)),   # several chunks: the jump sits in the last prefix tile
])
@BESIDE
def test_attention_large_score_jump(B, lens, boost_rows, beside):
    """Scores that jump far above everything seen before in a chunk (a few keys scaled by
    40): the softmax reference of the first tiles would overflow, so the kernel has to take
    its second pass from the true chunk max; the result must still match the oracle."""
    require_gpu()
    wl = _bf16(branching_tree((4, 3, 2, 1)), B, 32, 8, 128, max(lens))
    x = W.gen_attention(wl, 61, np.asarray(lens, np.int32))
    lo, hi = boost_rows
    x["k_cache"][0, :, lo:hi] = W.round_bf16(x["k_cache"][0, :, lo:hi] * np.float32(40.0))
    dt = torch.bfloat16
    anc = ops.build_tree_mask(dev_i32(wl.parents))["anc_mask"]
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    out, lse = ops.tree_attn_verify(dev(x["q"], dt), dev(x["k_cache"], dt), dev(x["v_cache"], dt),
                                    dev_i32(x["prefix_len"]), anc, max(lens), status=status,
                                    beside=beside)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    rng = np.random.default_rng(62)
    sel = [(b, int(rng.integers(32)), int(rng.integers(64))) for b in range(B) for _ in range(12)]
    ref = O.tree_attention(x["q"], x["k_cache"], x["v_cache"], x["prefix_len"],
                           O.build_tree(list(wl.parents))["anc"], select=sel)
    bb, hh, ii = np.array(sel).T
    s_max = float(np.max(ref["lse"][bb, hh, ii]))
    print(f"largest selected lse {s_max:.1f} (natural log units)")
    assert s_max > 64 * np.log(2.0)   # the jump really exceeds the first-pass slack
    assert_bf16(host(out)[bb, ii, hh], ref["out"][bb, ii, hh], what="out")
    assert_fp32(host(lse)[bb, hh, ii], ref["lse"][bb, hh, ii], atol=1e-3, what="lse")


@BESIDE
def test_attention_bad_prefix_flags(beside):
    require_gpu()
    wl = _bf16([-1, 0], 2, 4, 2, 64, 10)
    x = W.gen_attention(wl, 5, np.array([10, 10], np.int32))
    anc = ops.build_tree_mask(dev_i32(wl.parents))["anc_mask"]
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    pl = dev_i32([10, 50])                 # 50 > max_L and 50 + N > L_cap
    ops.tree_attn_verify(dev(x["q"], torch.bfloat16), dev(x["k_cache"], torch.bfloat16),
                         dev(x["v_cache"], torch.bfloat16), pl, anc, 10, status=status,
                         beside=beside)
    torch.cuda.synchronize()
    assert int(status.item()) & L.MV_DEV_BAD_PREFIX
