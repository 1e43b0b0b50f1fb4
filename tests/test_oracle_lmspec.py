"""Pins of oracle.accept_speculative_lm: the speculative rule with the target distribution from
an LM head (softmax of W_lm x_t) and the draft distribution of depth k from draft logits row k.

Pins: a hand-worked chain over a 3-token vocabulary (every probability, alpha, residual and the
drawn token written out as fractions; it fixes which target row (the parent's) and which draft
row (the node's depth) a test uses); uniform target and draft (everything accepted, extra token
floor(u V)); a draft with all its mass on one token (that token's node accepted iff u < 1/V,
the residual uniform over the other tokens)."""
import numpy as np

from oracle import medusa_oracle as O


def test_hand_worked_chain():
    # W_lm rows: token 0 reads x[0], token 1 reads x[1], token 2 reads nothing (logit 0)
    w = np.array([[1.0, 0.0], [0.0, 1.0], [0.0, 0.0]])
    x_t = np.array([[[np.log(2.0), 0.0],      # row 0 (after the prefix): P_t = [1/2, 1/4, 1/4]
                     [0.0, np.log(3.0)],      # row 1 (after node 0):     P_t = [1/5, 3/5, 1/5]
                     [0.0, 0.0]]])            # row 2 (after node 1):     uniform
    draft = np.array([[[0.0, 0.0, 0.0],       # depth 1: P_d = [1/3, 1/3, 1/3]
                       [np.log(4.0), 0.0, 0.0]]])  # depth 2: P_d = [4/6, 1/6, 1/6]
    parents = [-1, 0]
    tokens = np.array([[0, 0]])
    u = np.array([[0.9, 0.5, 0.95]])
    r = O.accept_speculative_lm(x_t, w, draft, tokens, parents, u, 2)
    # node 0: P_t = 1/2 (row 0) vs P_d = 1/3 (depth 1): alpha 1, accepted (0.9 < 1)
    # node 1: P_t = 1/5 (row 1) vs P_d = 4/6 (depth 2): alpha 3/10, rejected (0.5)
    np.testing.assert_allclose(r["alpha"][0], [1.0, 0.3], rtol=0, atol=1e-12)
    assert r["accept_len"][0] == 1 and list(r["path_nodes"][0]) == [0, -1]
    # residual at row 1: max(0, [1/5 - 4/6, 3/5 - 1/6, 1/5 - 1/6]) = [0, 13/30, 1/30] -> CDF
    # [0, 13/14, 1]; u = 0.95 first exceeded at token 2
    assert list(r["out_tokens"][0]) == [0, 2, -1]
    u2 = np.array([[0.9, 0.5, 0.9]])       # 0.9 < 13/14: token 1
    assert list(O.accept_speculative_lm(x_t, w, draft, tokens, parents, u2, 2)["out_tokens"][0]) == [0, 1, -1]


def test_uniform_target_and_draft_accept_everything():
    B, V, d, N = 2, 7, 4, 6
    parents = [-1, 0, 1, -1, 3, 4]          # two chains of depth 3
    tokens = np.array([[0, 1, 2, 3, 4, 5], [6, 5, 4, 3, 2, 1]])
    x_t = np.zeros((B, N + 1, d))
    w = np.zeros((V, d))                    # all logits 0: P_t uniform
    draft = np.zeros((B, 3, V))             # P_d uniform at every depth
    u = np.array([[0.3, 0.9, 0.1, 0.2, 0.99, 0.4, 0.55], [0.0, 0.5, 0.5, 0.5, 0.5, 0.5, 0.999]])
    r = O.accept_speculative_lm(x_t, w, draft, tokens, parents, u, 3)
    assert np.all(r["alpha"] == 1.0)
    np.testing.assert_array_equal(r["accept_len"], [3, 3])
    np.testing.assert_array_equal(r["path_nodes"], [[0, 1, 2], [0, 1, 2]])   # first longest
    # a leaf terminal: the extra token comes from P_t (uniform): floor(u V)
    assert r["out_tokens"][0][3] == int(np.floor(0.55 * V))
    assert r["out_tokens"][1][3] == int(np.floor(0.999 * V))


def test_draft_concentrated_on_one_token():
    V, d = 5, 3
    w = np.zeros((V, d))                    # uniform target: 1/5 everywhere
    draft = np.zeros((1, 1, V))
    draft[0, 0, 2] = 60.0                   # P_d(2) ~ 1, the others ~ e^-60
    parents = [-1, -1]
    tokens = np.array([[2, 4]])             # node 0 proposes the draft's token, node 1 another
    x_t = np.zeros((1, 3, d))
    # alpha(node 0) = (1/5) / ~1 = 1/5; alpha(node 1) = 1 (P_d tiny)
    r = O.accept_speculative_lm(x_t, w, draft, tokens, parents, np.array([[0.19, 0.5, 0.0]]), 1)
    np.testing.assert_allclose(r["alpha"][0], [0.2, 1.0], rtol=1e-12)
    assert list(r["node_accept"][0]) == [True, True] and r["path_nodes"][0][0] == 0
    r = O.accept_speculative_lm(x_t, w, draft, tokens, parents, np.array([[0.21, 0.7, 0.0]]), 1)
    assert r["accept_len"][0] == 1 and r["path_nodes"][0][0] == 1      # node 0 rejected
    # both rejected is impossible here (alpha 1 for node 1), so test the residual with one node
    r = O.accept_speculative_lm(x_t[:, :2], w, draft, tokens[:, :1], [-1], np.array([[0.5, 0.0]]), 1)
    assert r["accept_len"][0] == 0
    # residual at row 0: max(0, 1/5 - P_d) = 1/5 on tokens 0, 1, 3, 4 and 0 on token 2;
    # u = 0 draws the first positive one
    assert r["out_tokens"][0][0] == 0
    r = O.accept_speculative_lm(x_t[:, :2], w, draft, tokens[:, :1], [-1], np.array([[0.5, 0.6]]), 1)
    assert r["out_tokens"][0][0] == 3       # cumulative 1/4, 2/4, 3/4: 0.6 falls on token 3
