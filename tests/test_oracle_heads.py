"""Pins for the oracle's Medusa heads.

References: torch's functional linear/SiLU (the building blocks the page's own
PyTorch head uses, here without the residual-block bias the equation omits),
a W_res = 0 special case that reduces a head to one matrix-vector product,
scipy's logsumexp, and Python's sorted() for top-k.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F
from scipy.special import logsumexp

from oracle import medusa_oracle as O


def test_silu_matches_torch():
    x = np.linspace(-30, 30, 2001)
    np.testing.assert_allclose(O.silu(x), F.silu(torch.from_numpy(x)).numpy(), rtol=1e-14, atol=1e-300)
    assert O.silu(np.array([0.0]))[0] == 0.0


def test_heads_match_torch_functional():
    rng = np.random.default_rng(0)
    B, d, V, K = 3, 24, 57, 3
    h = rng.standard_normal((B, d))
    w_res = rng.standard_normal((K, d, d)) / np.sqrt(d)
    w_head = rng.standard_normal((K, V, d)) / np.sqrt(d)
    res = O.medusa_heads(h, w_res, w_head, widths=[4, 3, 1])
    th = torch.from_numpy(h)
    for k in range(K):
        hk = F.silu(F.linear(th, torch.from_numpy(w_res[k]))) + th
        logits = F.linear(hk, torch.from_numpy(w_head[k])).numpy()
        np.testing.assert_allclose(res["hk"][:, k], hk.numpy(), rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(res["logits"][:, k], logits, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(res["lse"][:, k], logsumexp(logits, axis=1), rtol=1e-13)


def test_zero_residual_weights_reduce_to_one_matvec():
    rng = np.random.default_rng(1)
    d, V = 16, 40          # V != d so a transposed operand cannot pass
    h = rng.standard_normal((2, d))
    w_head = rng.standard_normal((1, V, d))
    res = O.medusa_heads(h, np.zeros((1, d, d)), w_head, widths=[5])
    np.testing.assert_allclose(res["hk"][:, 0], h, rtol=0, atol=0)
    np.testing.assert_allclose(res["logits"][:, 0], h @ w_head[0].T, rtol=1e-13, atol=1e-13)


def test_topk_order_and_ties_by_sorted():
    rng = np.random.default_rng(2)
    for trial in range(50):
        V = int(rng.integers(1, 40))
        row = rng.integers(-3, 4, size=V).astype(np.float64)   # many ties
        s = int(rng.integers(1, V + 1))
        t = O.topk_rows(row, s)
        ref = [j for _, j in sorted(((-row[j], j) for j in range(V)))[:s]]
        assert t["ids"].tolist() == ref
        assert t["vals"].tolist() == [row[j] for j in ref]


def test_topk_of_probabilities_equals_topk_of_logits():
    rng = np.random.default_rng(3)
    d, V = 8, 100
    res = O.medusa_heads(rng.standard_normal((1, d)), rng.standard_normal((1, d, d)),
                         rng.standard_normal((1, V, d)), widths=[6])
    p = np.exp(res["logits"][0, 0] - res["lse"][0, 0])
    assert abs(p.sum() - 1) < 1e-12
    ref = [j for _, j in sorted((-p[j], j) for j in range(V))[:6]]
    assert res["topk_ids"][0, 0].tolist() == ref


def test_topk_padding_past_width():
    rng = np.random.default_rng(4)
    res = O.medusa_heads(rng.standard_normal((1, 4)), rng.standard_normal((2, 4, 4)),
                         rng.standard_normal((2, 9, 4)), widths=[3, 1])
    assert res["topk_ids"].shape == (1, 2, 3)
    assert res["topk_ids"][0, 1, 1:].tolist() == [-1, -1]
    assert np.all(np.isneginf(res["topk_vals"][0, 1, 1:]))
