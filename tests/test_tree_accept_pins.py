"""Pins of the oracle's tree acceptance (oracle/tree_accept.py) against what the LLM
Primer's section 9.1 and the mathematics fix, independently of the oracle's code: the
emitted token is distributed exactly as the target's (Monte Carlo, on a chain and on
sibling groups drawn without replacement), greedy longest match on a hand-worked tree,
and closed-form special cases."""
import numpy as np
import pytest

from oracle import tree_accept as TA


def _first_token(p, q, k, rng, trials):
    """Root with k children drafted from q without replacement; returns the empirical
    distribution of the first emitted token (the accepted child's, else the bonus)."""
    V = p.shape[0]
    counts = np.zeros(V)
    parent = np.full(k, -1, np.int32)
    for _ in range(trials):
        toks = rng.choice(V, size=k, replace=False, p=q)
        u = rng.random(k).astype(np.float32)
        ub = np.float32(rng.random())
        path, y, _ = TA.accept_tree(p, q, np.zeros((k, V)), np.zeros((k, V)), parent, toks, 0, k,
                                    u, ub, TA.SAMPLE, 8)
        counts[toks[path[0]] if path else y] += 1
    return counts / trials


@pytest.mark.parametrize("k,peaked", [(1, False), (2, False), (3, False), (2, True), (3, True)])
def test_sampling_preserves_the_target_distribution(k, peaked):
    """Primer section 9.1: accepting with min(1, p/q) and resampling from (p - q)+ leaves
    the output distributed as p. Here with k sibling drafts (k = 1 is the chain rule).
    The peaked case drafts mostly a token the target disfavours, so later siblings are
    tested against residuals from which a heavy token was removed: a rule that leaves
    the rejected token in q_res is off by several sigma there."""
    rng = np.random.default_rng(10 + k)
    V = 5
    if peaked:
        p = np.array([0.05, 0.3, 0.3, 0.2, 0.15])
        q = np.array([0.6, 0.1, 0.1, 0.1, 0.1])
    else:
        p = rng.dirichlet(np.ones(V)).astype(np.float32).astype(np.float64)
        q = rng.dirichlet(np.ones(V)).astype(np.float32).astype(np.float64)
    p /= p.sum()
    q /= q.sum()
    N = 40000
    f = _first_token(p, q, k, rng, N)
    sigma = np.sqrt(p * (1 - p) / N)
    assert np.all(np.abs(f - p) < 5 * sigma + 1e-4), (f, p)


def test_greedy_hand_worked_tree():
    """Context argmax is token 2; children carry tokens 1 and 2, so child 1 is accepted.
    Its argmax is token 3, carried by its child (node 2): accepted. Node 2's argmax is
    token 0, carried by no child: the bonus token is 0."""
    V = 4
    p_ctx = np.array([0.1, 0.2, 0.6, 0.1], np.float32)
    parent = np.array([-1, -1, 1, 1], np.int32)
    token = np.array([1, 2, 3, 0], np.int32)
    p_node = np.array([[0.9, 0.1, 0, 0], [0.1, 0.1, 0.3, 0.5], [0.7, 0.1, 0.1, 0.1],
                       [0.25, 0.25, 0.25, 0.25]], np.float32)
    path, y, _ = TA.accept_tree(p_ctx, None, p_node, None, parent, token, 0, 4, None, 0.5,
                                TA.GREEDY, 8)
    assert path == [1, 2] and y == 0
    # ties go to the lowest token id: node 3's row is flat -> token 0
    path, y, _ = TA.accept_tree(np.array([0, 0, 0, 1], np.float32), None, p_node, None, parent,
                                token, 0, 4, None, 0.5, TA.GREEDY, 8)
    assert path == [] and y == 3


def test_equal_distributions_always_accept_the_first_child():
    rng = np.random.default_rng(3)
    V, n = 6, 5
    parent = np.array([-1, 0, 0, 1, -1], np.int32)
    token = np.array([2, 4, 1, 0, 3], np.int32)
    rows = rng.dirichlet(np.ones(V), size=n).astype(np.float32)
    ctx = rng.dirichlet(np.ones(V)).astype(np.float32)
    for _ in range(20):
        u = rng.random(n).astype(np.float32) * np.float32(0.999)
        path, y, _ = TA.accept_tree(ctx, ctx, rows, rows, parent, token, 0, n, u, 0.3,
                                    TA.SAMPLE, 8)
        assert path == [0, 1, 3]


def test_disjoint_draft_always_rejects_and_resamples_the_target():
    """q puts all its mass on a token the target never picks: every draft is rejected,
    the residual (p - q)+ normalised is p itself, so the bonus follows p (checked by
    inverse CDF on a grid of uniforms)."""
    V = 4
    p = np.array([0.5, 0.3, 0.2, 0.0], np.float32)
    q = np.array([0.0, 0.0, 0.0, 1.0], np.float32)
    parent = np.array([-1], np.int32)
    token = np.array([3], np.int32)
    hits = np.zeros(V)
    grid = (np.arange(1000) + 0.5) / 1000
    for ub in grid:
        path, y, _ = TA.accept_tree(p, q, np.zeros((1, V)), np.zeros((1, V)), parent, token, 0,
                                    1, np.array([0.0], np.float32), ub, TA.SAMPLE, 8)
        assert path == []
        hits[y] += 1
    np.testing.assert_allclose(hits / 1000, p, atol=2e-3)


def test_max_path_truncates_the_walk():
    V = 3
    parent = np.array([-1, 0, 1], np.int32)
    token = np.array([0, 0, 0], np.int32)
    p = np.array([[1, 0, 0]] * 3, np.float32)
    path, y, _ = TA.accept_tree(np.array([1, 0, 0], np.float32), None, p, None, parent, token,
                                0, 3, None, 0.5, TA.GREEDY, 2)
    assert path == [0, 1] and y == 0


def test_batch_statuses():
    V = 4
    parent = np.array([-1, 0, -1, 1, -1, 0], np.int32)     # tree 1: node 1 is its own parent
    token = np.array([0, 1, 2, 3, 9, 0], np.int32)           # tree 2: token 9 is outside V
    offs = np.array([0, 2, 4, 6], np.int32)
    rows = np.full((6, V), 0.25, np.float32)
    ctx = np.full((3, V), 0.25, np.float32)
    r = TA.accept_trees(ctx, ctx, rows, rows, parent, token, offs, np.zeros(6, np.float32),
                        np.full(3, 0.5, np.float32), TA.SAMPLE, 4)
    assert r["status"].tolist() == [TA.TREE_OK, TA.TREE_BAD_PARENT, TA.TREE_BAD_TOKEN]
    assert r["bonus"].tolist()[1:] == [-1, -1] and r["accepted_len"].tolist()[1:] == [0, 0]
    bad = TA.accept_trees(ctx, ctx, rows, rows, parent, token, np.array([0, 4, 2, 6], np.int32),
                          np.zeros(6, np.float32), np.full(3, 0.5, np.float32), TA.SAMPLE, 4)
    assert bad["status"].tolist()[1] == TA.TREE_BAD_SIZE
