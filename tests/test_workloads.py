"""Input generator: determinism, shapes, bf16 exactness, tree shapes."""
import numpy as np

from medusa_tree_attention_verify_amd import workloads as W


def test_named_trees():
    assert W.WORKLOADS["c1"].parents == (-1, -1, 0, 1, 2, 3, 4, 5)
    assert W.WORKLOADS["c2"].N == 64 and W.WORKLOADS["c4"].N == 212
    t = W.branching_tree((4, 3, 2, 1))
    assert t[4:7] == [0, 0, 0] and t[16:18] == [4, 4] and t[40] == 16


def test_block_seeding_is_thread_independent_and_deterministic():
    a = W.normal(5, "x", (3, 1 << 21), 0.5)
    b = W.normal(5, "x", (3, 1 << 21), 0.5)
    assert np.array_equal(a, b)
    assert not np.array_equal(a, W.normal(6, "x", (3, 1 << 21), 0.5))
    assert abs(a.std() - 0.5) < 0.01


def test_bf16_round_trip():
    x = W.normal(1, "y", (1000,), 3.0, bf16=True)
    bits = W.bf16_bits(x)
    back = (bits.astype(np.uint32) << 16).view(np.float32)
    assert np.array_equal(back, x)
    # ties to even: 1 + 2^-8 lies halfway between 1 and 1 + 2^-7 -> rounds to 1
    assert W.round_bf16(np.array([1 + 2 ** -8], np.float32))[0] == 1.0
    assert W.round_bf16(np.array([1 + 3 * 2 ** -8], np.float32))[0] == 1 + 2 ** -6


def test_small_workload_shapes():
    wl = W.WORKLOADS["c1"]
    heads = W.gen_heads(wl, 1)
    assert heads["w_head"].shape == (3, 1000, 256)
    att = W.gen_attention(wl, 1)
    assert att["k_cache"].shape == (1, 4, 136, 64) and att["L_cap"] == 136
    wl5 = W.WORKLOADS["c5"].scaled(B=2, accept_V=300)
    sp = W.gen_speculative(wl5, 1)
    assert sp["p_target"].shape == (2, 65, 300)
    np.testing.assert_allclose(sp["p_target"].sum(-1), 1, rtol=1e-5)
    # children of the prefix row propose the draft's top-4 tokens of row 0
    top = np.argsort(-sp["p_draft"][0, 0], kind="stable")[:4]
    assert sp["node_tokens"][0, :4].tolist() == top.tolist()
