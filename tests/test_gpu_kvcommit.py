"""GPU parity of the commit of the accepted path (mv_kv_commit) against the oracle: a copy, so
every comparison is bit-exact."""
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


def _random_paths(parents, B, D, seed):
    """One root path per sequence (of a random node, so of random length 1..depth, or empty
    for every fourth sequence), padded with zeros to D."""
    rng = W.rng_for(seed, "commit_paths")
    path_nodes = np.zeros((B, D), dtype=np.int32)
    alen = np.zeros(B, dtype=np.int32)
    for b in range(B):
        if b % 4 == 3:
            continue
        p = []
        c = int(rng.integers(0, len(parents)))
        while c != -1:
            p.append(c)
            c = parents[c]
        p = p[::-1][:D]
        path_nodes[b, :len(p)] = p
        alen[b] = len(p)
    return path_nodes, alen


def _bits(t):
    """Bit pattern of a device tensor on the host (bit-exact comparison, NaN-safe)."""
    t = t.detach().cpu()
    return (t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)).numpy()


@pytest.mark.parametrize("dtype,dh", [("bf16", 128), ("bf16", 64), ("f32", 128), ("f32", 64)])
def test_commit_small(dtype, dh):
    require_gpu()
    parents = branching_tree((4, 3, 2, 1))
    N, B, Hkv = len(parents), 9, 3
    D = int(O.build_tree(parents)["depth"].max())
    print(f"kv commit {dtype} dh={dh} B={B} Hkv={Hkv} N={N} D={D}", flush=True)
    bf = dtype == "bf16"
    prefix = W.rng_for(3, "commit_prefix").integers(0, 50, B).astype(np.int32)
    L_cap = int(prefix.max()) + N + 5
    k = W.normal(4, "commit_k", (B, Hkv, L_cap, dh), 1.0, bf)
    v = W.normal(4, "commit_v", (B, Hkv, L_cap, dh), 1.0, bf)
    path_nodes, alen = _random_paths(parents, B, D, 5)
    path_nodes[0, :2] = [1, 8]              # 1 -> 8 overlaps: row L+1 is read and written
    alen[0] = 2
    assert parents[8] == 1
    tdt = torch.bfloat16 if bf else torch.float32
    kd, vd, pd = dev(k, tdt), dev(v, tdt), dev_i32(prefix)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    ops.kv_commit(kd, vd, pd, N, dev_i32(path_nodes), dev_i32(alen), status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    k2, v2, p2 = O.kv_commit(k, v, prefix, path_nodes, alen, N)
    np.testing.assert_array_equal(host(pd), p2)
    np.testing.assert_array_equal(_bits(kd), _bits(torch.from_numpy(k2).to(tdt)))
    np.testing.assert_array_equal(_bits(vd), _bits(torch.from_numpy(v2).to(tdt)))


def test_commit_invalid_paths_leave_sequence_unchanged():
    require_gpu()
    N, B, Hkv, dh, D = 6, 4, 2, 64, 3
    L_cap = 20
    k = W.normal(6, "commit_k", (B, Hkv, L_cap, dh), 1.0, True)
    prefix = np.array([3, 3, 3, 15], dtype=np.int32)      # sequence 3: 15 + 6 > 20
    path_nodes = np.array([[0, 0, 0], [0, 2, 3], [0, 9, 0], [0, 1, 0]], dtype=np.int32)
    alen = np.array([2, 3, 2, 1], dtype=np.int32)         # seq 0: node 0 on level 1
    kd, vd, pd = dev(k, torch.bfloat16), dev(-k, torch.bfloat16), dev_i32(prefix)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    pout = torch.full((B,), -7, dtype=torch.int32, device="cuda")    # a separate output
    ops.kv_commit(kd, vd, pd, N, dev_i32(path_nodes), dev_i32(alen), status, prefix_out=pout)
    torch.cuda.synchronize()
    assert int(status.item()) == L.MV_DEV_BAD_PATH | L.MV_DEV_BAD_PREFIX
    np.testing.assert_array_equal(host(pd), prefix)                     # input kept
    # only sequence 1 is valid
    ok = np.array([1])
    k2, v2, p2 = O.kv_commit(k[ok], -k[ok], prefix[ok], path_nodes[ok], alen[ok], N)
    got_k = host(kd)
    np.testing.assert_array_equal(host(pout), [3, 6, 3, 15])
    np.testing.assert_array_equal(got_k[1], k2[0])
    np.testing.assert_array_equal(host(vd)[1], v2[0])
    for b in (0, 2, 3):
        np.testing.assert_array_equal(got_k[b], k[b])


@pytest.mark.parametrize("name", ["c2", "c5"])
def test_commit_full_size(name):
    """At the full cache sizes (Llama-3-8B layer: 4096 + 64 rows; 64 serving sequences with
    prefixes up to 8192): the oracle commits each sequence's tree block, the rest of the cache
    must be untouched."""
    require_gpu()
    wl = W.WORKLOADS[name]
    parents = list(wl.parents)
    N, B, Hkv, dh = wl.N, wl.B, wl.Hkv, wl.dh
    D = int(O.build_tree(parents)["depth"].max())
    prefix = W.gen_prefix_lens(wl, 11)
    L_cap = int(prefix.max()) + N
    print(f"kv commit full {name} B={B} L_cap={L_cap}", flush=True)
    g = torch.Generator(device="cuda").manual_seed(11)
    kd = torch.randn((B, Hkv, L_cap, dh), generator=g, device="cuda").to(torch.bfloat16)
    vd = torch.randn((B, Hkv, L_cap, dh), generator=g, device="cuda").to(torch.bfloat16)
    k0, v0 = kd.clone(), vd.clone()
    path_nodes, alen = _random_paths(parents, B, D, 12)
    pd = dev_i32(prefix)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    ops.kv_commit(kd, vd, pd, N, dev_i32(path_nodes), dev_i32(alen), status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    np.testing.assert_array_equal(host(pd), prefix + alen)
    for b in range(B):
        Lb = int(prefix[b])
        blk = slice(Lb, Lb + N)
        kb, vb = host(k0[b:b + 1, :, blk]), host(v0[b:b + 1, :, blk])
        k2, v2, _ = O.kv_commit(kb, vb, np.zeros(1, np.int32), path_nodes[b:b + 1],
                                alen[b:b + 1], N)
        np.testing.assert_array_equal(host(kd[b:b + 1, :, blk]), k2)
        np.testing.assert_array_equal(host(vd[b:b + 1, :, blk]), v2)
        assert torch.equal(kd[b, :, :Lb], k0[b, :, :Lb]) and torch.equal(vd[b, :, :Lb], v0[b, :, :Lb])
        assert torch.equal(kd[b, :, Lb + N:], k0[b, :, Lb + N:])


def test_verify_commit_verify():
    """Two verification steps on the GPU (fp32): tree attention, commit of a path per
    sequence, then a chain of the path's queries over the committed cache from the new
    prefix's start.  The second pass must reproduce the oracle's first-pass outputs of the
    path's nodes: the committed rows continue the prefix causally."""
    require_gpu()
    parents = list(W.WORKLOADS["c1"].parents)
    N, B = len(parents), 3
    wl = W.Workload(name="commit-loop", dtype="f32", B=B, Hq=8, Hkv=2, dh=64,
                    parents=tuple(parents), prefix=(40, 300), depth_widths=(1,))
    D = int(O.build_tree(parents)["depth"].max())
    x = W.gen_attention(wl, 13)
    anc = O.build_tree(parents)["anc"]
    qd, kd, vd = dev(x["q"]), dev(x["k_cache"]), dev(x["v_cache"])
    pd = dev_i32(x["prefix_len"])
    path_nodes, alen = _random_paths(parents, B, D, 14)     # B < 4: no empty path
    ref = O.tree_attention(x["q"], x["k_cache"], x["v_cache"], x["prefix_len"], anc)
    mask = ops.build_tree_mask(dev_i32(parents))["anc_mask"]
    max_L = int(x["prefix_len"].max())
    out1, _ = ops.tree_attn_verify(qd, kd, vd, pd, mask, max_L)
    ops.kv_commit(kd, vd, pd, N, dev_i32(path_nodes), dev_i32(alen))
    # second pass: chain over the kept rows, queried from the old prefix end
    chain = ops.build_tree_mask(dev_i32([-1] + list(range(D - 1))))["anc_mask"]
    qc = torch.zeros((B, D, wl.Hq, wl.dh), device="cuda")
    for b in range(B):
        qc[b, :alen[b]] = qd[b, path_nodes[b, :alen[b]].tolist()]
    p_old = dev_i32(x["prefix_len"])
    out2, lse2 = ops.tree_attn_verify(qc, kd, vd, p_old, chain, max_L)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(pd), x["prefix_len"] + alen)
    o1, o2 = host(out1), host(out2)
    for b in range(B):
        nodes = path_nodes[b, :alen[b]]
        assert_fp32(o1[b, nodes], ref["out"][b, nodes], what="first pass")
        assert_fp32(o2[b, :alen[b]], ref["out"][b, nodes], what="after commit")
        assert_fp32(host(lse2)[b, :, :alen[b]], ref["lse"][b][:, nodes], what="lse after commit")


def test_decode_loop_three_steps():
    """Three verify steps in a row (fp32), each ending with the commit: every step writes a
    fresh tree's K/V after the current prefix, verifies it, accepts greedily and commits, and
    the next step starts from the grown prefix.  The oracle runs the same loop on the host;
    attention, acceptance, the cache and the prefix lengths are compared at every step."""
    require_gpu()
    from medusa_tree_attention_verify_amd.step import VerifyStep
    parents = branching_tree((3, 2, 1))
    N, B, Hq, Hkv, dh, V = len(parents), 4, 8, 2, 64, 50
    D = 3
    anc = O.build_tree(parents)["anc"]
    prefix = np.array([5, 17, 30, 0], dtype=np.int64)
    L_cap = int(prefix.max()) + 3 * D + N
    kh = W.normal(40, "loop_k", (B, Hkv, L_cap, dh))
    vh = W.normal(40, "loop_v", (B, Hkv, L_cap, dh))
    kd, vd = dev(kh), dev(vh)
    pd = dev_i32(prefix)
    step = VerifyStep(parents=parents, depth_widths=(3, 2, 1), dtype=torch.float32, B=B, Hq=Hq,
                      Hkv=Hkv, dh=dh, max_L=L_cap - N, accept="greedy", V=V,
                      tokens_given=True, commit=True)
    total = 0
    for s in range(3):
        print(f"decode loop step {s} prefix {prefix.tolist()}", flush=True)
        q = W.normal(41 + s, "loop_q", (B, N, Hq, dh))
        newk = W.normal(41 + s, "loop_tree_k", (B, Hkv, N, dh))
        newv = W.normal(41 + s, "loop_tree_v", (B, Hkv, N, dh))
        for b in range(B):
            Lb = int(prefix[b])
            kh[b, :, Lb:Lb + N] = newk[b]
            vh[b, :, Lb:Lb + N] = newv[b]
            kd[b, :, Lb:Lb + N] = dev(newk[b])
            vd[b, :, Lb:Lb + N] = dev(newv[b])
        toks = W.rng_for(41 + s, "loop_tokens").integers(0, V, (B, N)).astype(np.int32)
        target = W.plant_greedy(W.normal(41 + s, "loop_target", (B, N + 1, V), 2.0),
                                parents, toks, 41 + s, 0.7)
        inp = {"q": dev(q), "k_cache": kd, "v_cache": vd, "prefix_len": pd,
               "target": dev(target), "node_tokens": dev_i32(toks)}
        step.run(inp)
        torch.cuda.synchronize()
        assert int(step.status.item()) == 0
        ref = O.tree_attention(q, kh, vh, prefix, anc)
        assert_fp32(host(step.attn_out), ref["out"], what=f"attention, step {s}")
        acc = O.accept_greedy(target, toks, parents, D)
        for k in ("accept_len", "path_nodes", "out_tokens"):
            np.testing.assert_array_equal(host(step.acc[k]), acc[k], err_msg=f"{k}, step {s}")
        kh, vh, prefix = O.kv_commit(kh, vh, prefix, acc["path_nodes"], acc["accept_len"], N)
        np.testing.assert_array_equal(host(step.prefix_next), prefix)
        np.testing.assert_array_equal(host(kd), kh)
        np.testing.assert_array_equal(host(vd), vh)
        pd.copy_(step.prefix_next)
        total += int(acc["accept_len"].sum())
    print("accepted tokens over 3 steps:", total)
    assert total > 0
