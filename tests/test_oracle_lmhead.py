"""Pins for the oracle's target LM head (greedy token, its logit and LSE per row).

References: closed forms that hold for special weights (all-zero W, a W with a single non-zero
row, unit-norm rows that make Cauchy-Schwarz decide the argmax), torch's functional linear
and scipy's logsumexp on a random case, and the page's greedy rule fed through the acceptance
oracle.
"""
import numpy as np
import torch
import torch.nn.functional as F
from scipy.special import logsumexp

from oracle import medusa_oracle as O


def test_zero_weights_tie_to_token_zero_and_log_v():
    x = np.random.default_rng(0).standard_normal((3, 16))
    r = O.lm_head_argmax(x, np.zeros((37, 16)))
    assert r["ids"].tolist() == [0, 0, 0]          # every logit ties: lowest id
    np.testing.assert_array_equal(r["max"], 0.0)
    np.testing.assert_allclose(r["lse"], np.log(37.0), rtol=0, atol=1e-15)


def test_single_nonzero_row_closed_form():
    rng = np.random.default_rng(1)
    d, V = 8, 50
    x = rng.standard_normal((1, d)) * 0.5
    w = np.zeros((V, d))
    w[23] = x[0]
    r = O.lm_head_argmax(x, w)
    q = float(x[0] @ x[0])
    assert r["ids"][0] == 23
    np.testing.assert_allclose(r["max"][0], q, rtol=1e-15)
    np.testing.assert_allclose(r["lse"][0], np.log((V - 1) + np.exp(q)), rtol=1e-14)


def test_unit_rows_pick_their_own_row():
    """W's first T rows are the unit-norm hidden states themselves (rest random, smaller):
    by Cauchy-Schwarz row t's logits peak at v = t.  A transposed product (x^T W) or a
    row/column mix-up fails this."""
    rng = np.random.default_rng(2)
    T, d, V = 6, 32, 40
    x = rng.standard_normal((T, d))
    x /= np.linalg.norm(x, axis=1, keepdims=True)
    w = rng.standard_normal((V, d)) * 0.01
    w[:T] = x
    r = O.lm_head_argmax(x, w)
    assert r["ids"].tolist() == list(range(T))


def test_random_case_matches_torch_and_scipy():
    rng = np.random.default_rng(3)
    T, d, V = 5, 48, 301
    x = rng.standard_normal((T, d))
    w = rng.standard_normal((V, d)) / np.sqrt(d)
    r = O.lm_head_argmax(x, w)
    z = F.linear(torch.from_numpy(x), torch.from_numpy(w)).numpy()
    np.testing.assert_allclose(r["logits"], z, rtol=1e-12, atol=1e-12)
    assert r["ids"].tolist() == [int(np.flatnonzero(row == row.max())[0]) for row in z]
    np.testing.assert_allclose(r["lse"], logsumexp(z, axis=1), rtol=1e-13)
    # P_target = exp(z - LSE) is a distribution
    np.testing.assert_allclose(np.exp(z - r["lse"][:, None]).sum(axis=1), 1.0, rtol=1e-13)


def test_greedy_acceptance_from_lm_head():
    """The page's greedy rule on LM-head outputs: plant the tree tokens so that the chain
    0 -> 1 matches the target's greedy tokens and node 2 does not; acceptance stops there."""
    rng = np.random.default_rng(4)
    d, V = 16, 30
    parents = [-1, 0, 1]
    x = rng.standard_normal((1, 4, d))
    w = rng.standard_normal((V, d))
    r = O.lm_head_argmax(x[0], w)
    g = r["ids"]                       # rows 0..3: after the prefix, after node 0, 1, 2
    toks = np.array([[g[0], g[1], (g[2] + 1) % V]], dtype=np.int64)
    out = O.accept_greedy(r["logits"][None], toks, parents, D=3)
    assert int(out["accept_len"][0]) == 2
    assert out["out_tokens"][0].tolist()[:3] == [g[0], g[1], g[2]]   # 2 accepted + bonus
