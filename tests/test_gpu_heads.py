"""GPU parity of the Medusa heads (residual block + projection/top-k/LSE) and of mv_topk_rows."""
import numpy as np
import pytest
import torch

from oracle import medusa_oracle as O
from medusa_tree_attention_verify_amd import ops
from medusa_tree_attention_verify_amd import workloads as W
from tests.gpu_util import (assert_bf16, assert_fp32, check_topk, dev, host, require_gpu)

pytestmark = pytest.mark.gpu


def _run_and_check(wl, seed, widths, check_logits=True):
    x = W.gen_heads(wl, seed)
    dt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    h, w_res, w_head = dev(x["h"], dt), dev(x["w_res"], dt), dev(x["w_head"], dt)
    print(f"heads {wl.name} B={wl.B} d={wl.d} V={wl.V} K={wl.K} seed={seed}", flush=True)
    got = ops.medusa_heads(h, w_res, w_head, widths, want_hk=True, want_logits=check_logits)
    torch.cuda.synchronize()
    ref = O.medusa_heads(x["h"], x["w_res"], x["w_head"], widths)
    # fp32 outputs: h_k, top-k values, lse (LSE bound 1e-3 for bf16 inputs)
    assert_fp32(host(got["hk"]), ref["hk"], what="hk")
    lse_tol = 1e-4 if wl.dtype == "f32" else 1e-3
    assert_fp32(host(got["lse"]), ref["lse"], atol=lse_tol, what="lse")
    ties = check_topk(host(got["topk_ids"]), ref["logits"], widths)
    ids = host(got["topk_ids"])
    vals = host(got["topk_vals"])
    for b in range(wl.B):
        for k in range(wl.K):
            s = widths[k]
            assert_fp32(vals[b, k, :s], ref["logits"][b, k][ids[b, k, :s]], what="topk_vals")
            assert np.all(np.isneginf(vals[b, k, s:]))
    if check_logits:
        if wl.dtype == "f32":
            assert_fp32(host(got["logits"]), ref["logits"], what="logits")
        else:
            # bf16 logits: the kernel rounds its fp32 sum once; compare to the fp64 definition
            assert_bf16(host(got["logits"]), ref["logits"], what="logits")
    return ties


def test_heads_tiny_fp32():
    require_gpu()
    wl = W.WORKLOADS["c1"]
    assert _run_and_check(wl, 1, list(wl.head_widths)) == 0


@pytest.mark.parametrize("B", [1, 3, 8, 12, 20, 33, 40, 64])  # 33-64: eight column tiles
def test_heads_bf16_small(B):
    require_gpu()
    wl = W.WORKLOADS["c2"].scaled(B=B, d=256, V=1000, K=3, head_widths=(4, 3, 1))
    ties = _run_and_check(wl, 100 + B, [4, 3, 1])
    assert ties <= 1


@pytest.mark.parametrize("B,V,widths", [(3, 3000, (12, 9)),          # tournament, 16 per thread
                                         (1, 32000, (16, 10, 5)),     # tournament, 32 per thread
                                         (2, 64000, (16, 11))])       # 16-slot sorted lists
def test_heads_wide_candidate_lists(B, V, widths):
    """More than 8 candidates per head: the selection paths for long lists (d = 256)."""
    require_gpu()
    wl = W.WORKLOADS["c2"].scaled(B=B, d=256, V=V, K=len(widths), head_widths=widths)
    ties = _run_and_check(wl, 40 + B, list(widths), check_logits=False)
    assert ties <= 1


def test_heads_fp32_batched():
    require_gpu()
    wl = W.WORKLOADS["c1"].scaled(B=5, d=128, V=777, K=2, head_widths=(3, 2))
    _run_and_check(wl, 7, [3, 2])


def test_heads_fp32_large_vocab():
    """fp32 heads over 4 x 32000 rows (d = 64): enough row blocks that the projection runs
    4 waves per workgroup, so each wave takes two groups of rows."""
    require_gpu()
    wl = W.WORKLOADS["c1"].scaled(B=1, d=64, V=32000, K=4, head_widths=(4, 3, 2, 1))
    _run_and_check(wl, 9, [4, 3, 2, 1])


def test_heads_llama8b_shape_full():
    """d=4096, V=32000, 4 heads, widths (4,3,2,1), batch 1 (the full Llama-3-8B shape)."""
    require_gpu()
    wl = W.WORKLOADS["c2"]
    ties = _run_and_check(wl, 2, list(wl.head_widths), check_logits=True)
    print("near-tie ranks:", ties)
    assert ties <= 1


def test_heads_70b_width_batch8():
    """d=8192, batch 8 (the 70B one-GPU share's width and batch), vocabulary cut to 4000."""
    require_gpu()
    wl = W.WORKLOADS["c3"].scaled(V=4000)
    ties = _run_and_check(wl, 3, list(wl.head_widths), check_logits=True)
    print("near-tie ranks:", ties)
    assert ties <= 2


def test_heads_serving_batch64_sampled():
    """The Llama-3-8B head shape (d=4096, V=32000, 4 heads) at the serving batch of 64 (eight
    column tiles): the GPU computes every (batch row, head); the oracle recomputes sampled
    pairs, each from its own slice of the inputs."""
    require_gpu()
    wl = W.WORKLOADS["c2"].scaled(B=64)
    widths = list(wl.head_widths)
    x = W.gen_heads(wl, 29)
    print(f"heads B={wl.B} d={wl.d} V={wl.V} K={wl.K}", flush=True)
    got = ops.medusa_heads(dev(x["h"], torch.bfloat16), dev(x["w_res"], torch.bfloat16),
                           dev(x["w_head"], torch.bfloat16), widths, want_hk=True)
    torch.cuda.synchronize()
    hk, ids, vals, lse = (host(got[n]) for n in ("hk", "topk_ids", "topk_vals", "lse"))
    for b, k in ((0, 0), (17, 1), (40, 2), (63, 3), (63, 0)):
        ref = O.medusa_heads(x["h"][b:b + 1], x["w_res"][k:k + 1], x["w_head"][k:k + 1], [widths[k]])
        s = widths[k]
        assert_fp32(hk[b, k], ref["hk"][0, 0], what=f"hk b={b} k={k}")
        assert_fp32(lse[b, k], ref["lse"][0, 0], atol=1e-3, what=f"lse b={b} k={k}")
        ties = check_topk(ids[b:b + 1, k:k + 1], ref["logits"], [s])
        assert ties <= 1
        assert_fp32(vals[b, k, :s], ref["logits"][0, 0][ids[b, k, :s]], what=f"topk_vals b={b} k={k}")


def test_heads_70b_full_sampled():
    """The full 70B-share head shape (d=8192, V=32000, 4 heads, batch 8): the GPU computes every
    (batch row, head); the oracle recomputes four sampled pairs in fp64, each from its own slice
    of the same inputs, and their h_k, top-k ids/values and LSE must match."""
    require_gpu()
    wl = W.WORKLOADS["c3"]
    widths = list(wl.head_widths)
    x = W.gen_heads(wl, 13)
    print(f"heads full B={wl.B} d={wl.d} V={wl.V} K={wl.K}", flush=True)
    got = ops.medusa_heads(dev(x["h"], torch.bfloat16), dev(x["w_res"], torch.bfloat16),
                           dev(x["w_head"], torch.bfloat16), widths, want_hk=True)
    torch.cuda.synchronize()
    hk, ids, vals, lse = (host(got[n]) for n in ("hk", "topk_ids", "topk_vals", "lse"))
    for b, k in ((0, 0), (3, 1), (5, 2), (7, 3)):
        ref = O.medusa_heads(x["h"][b:b + 1], x["w_res"][k:k + 1], x["w_head"][k:k + 1], [widths[k]])
        s = widths[k]
        assert_fp32(hk[b, k], ref["hk"][0, 0], what=f"hk b={b} k={k}")
        assert_fp32(lse[b, k], ref["lse"][0, 0], atol=1e-3, what=f"lse b={b} k={k}")
        ties = check_topk(ids[b:b + 1, k:k + 1], ref["logits"], [s])
        assert ties <= 1
        assert_fp32(vals[b, k, :s], ref["logits"][0, 0][ids[b, k, :s]], what=f"topk_vals b={b} k={k}")


def test_split_calls_match_fused_and_repeat():
    """mv_medusa_residual + (mv_medusa_head_project + mv_medusa_head_select) twice equal
    mv_medusa_heads: they accumulate the same products in the same order."""
    require_gpu()
    wl = W.WORKLOADS["c2"].scaled(B=2, d=512, V=3000, K=4, head_widths=(4, 3, 2, 1))
    x = W.gen_heads(wl, 11)
    h, w_res, w_head = (dev(x[k], torch.bfloat16) for k in ("h", "w_res", "w_head"))
    widths = [4, 3, 2, 1]
    fused = ops.medusa_heads(h, w_res, w_head, widths, want_logits=True)
    ws = ops.Workspace()
    ops.medusa_residual(h, w_res, V=3000, s_max=4, ws=ws)
    runs = [ops.medusa_head_topk(w_head, 2, widths, lse=torch.empty((2, 4), device="cuda"),
                                 logits=torch.empty_like(fused["logits"]), ws=ws)
            for _ in range(2)]
    torch.cuda.synchronize()
    for r in runs:
        assert torch.equal(r["topk_ids"], fused["topk_ids"])
        assert torch.equal(r["topk_vals"], fused["topk_vals"])
        assert torch.equal(r["lse"], fused["lse"])
        assert torch.equal(r["logits"], fused["logits"])


@pytest.mark.parametrize("B,d", [(3, 800), (2, 96), (20, 2080)])
def test_projection_partial_stages(B, d):
    """The projection's row-segment loads stage 8 k-steps at a time per wave; widths whose
    per-wave k-range leaves a partial stage (d = 800, 2080) or no full stage (d = 96), with 1 to
    4 column tiles, against the oracle (logits, top-k, LSE)."""
    require_gpu()
    wl = W.WORKLOADS["c2"].scaled(B=B, d=d, V=1999)
    ties = _run_and_check(wl, 17, list(wl.head_widths), check_logits=True)
    assert ties <= 1


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("V,s", [(128256, 4), (131072, 16), (100003, 9)])
def test_topk_rows_long_rows(dtype, V, s):
    """Rows long enough for several load batches per thread, where elements below the wave's
    running threshold skip the insertion: integer rows (many exact ties across batches) and
    normal rows with their largest value planted again at scattered positions; ids, values
    and the row LSE against the oracle."""
    require_gpu()
    rng = np.random.default_rng(7 + V + s)
    x = np.empty((4, V), np.float32)
    x[:2] = rng.integers(-4, 5, size=(2, V))
    x[2:] = rng.standard_normal((2, V))
    if dtype == torch.bfloat16:
        x = W.round_bf16(x)
    for r in (2, 3):
        top = x[r].max()
        x[r, rng.choice(V, 5, replace=False)] = top
    print(f"topk rows V={V} s={s} {dtype}", flush=True)
    lse = torch.full((4,), float("nan"), dtype=torch.float32, device="cuda")
    ids, vals = ops.topk_rows(dev(x, dtype), s, lse=lse)
    torch.cuda.synchronize()
    for r in range(4):
        ref = O.topk_rows(x[r], s)
        np.testing.assert_array_equal(host(ids)[r], ref["ids"])
        np.testing.assert_array_equal(host(vals)[r], ref["vals"])
        # the row's LSE: the oracle's LM head over V one-column weight rows holding the row
        want = O.lm_head_argmax(np.ones((1, 1)), x[r][:, None])["lse"]
        assert_fp32(host(lse)[r:r + 1], want, atol=1e-4, what=f"row {r} lse")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("V,s", [(3001, 5), (3000, 4), (3000, 12)])  # scalar / 16-byte loads
def test_topk_rows_ties_and_strides(dtype, V, s):
    require_gpu()
    rng = np.random.default_rng(5 + V + s)
    R = 6
    x = rng.integers(-4, 5, size=(R, V)).astype(np.float32)   # many exact ties
    xt = dev(x, dtype)
    lse = torch.full((R,), float("nan"), dtype=torch.float32, device="cuda")
    ids, vals = ops.topk_rows(xt, s, lse=lse)
    torch.cuda.synchronize()
    for r in range(R):
        ref = O.topk_rows(x[r], s)
        np.testing.assert_array_equal(host(ids)[r], ref["ids"])
        np.testing.assert_array_equal(host(vals)[r], ref["vals"])
    # each row's log-sum-exp: the oracle's LM head with an identity weight has the rows as logits
    assert_fp32(host(lse), O.lm_head_argmax(x, np.eye(V))["lse"], atol=1e-4, what="row lse")
    # strided rows: every other row of a [2R, V] matrix, written with an output stride
    x2 = np.repeat(x, 2, axis=0)
    x2[1::2] = -100
    out = torch.full((R, 2 * s), -7, dtype=torch.int32, device="cuda")
    ops.topk_rows(dev(x2, dtype), s, R=R, V=V, ldx=2 * V, ids=out, vals=None, ld_out=2 * s)
    torch.cuda.synchronize()
    o = host(out)
    for r in range(R):
        np.testing.assert_array_equal(o[r, :s], O.topk_rows(x[r], s)["ids"])
        assert np.all(o[r, s:] == -7)
