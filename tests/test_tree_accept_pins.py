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


def test_two_rejections_hand_worked():
    """Exact rationals, worked by hand from the section 9.1 rule. p = (.3, .2, .3, .2),
    q = (.1, .5, .3, .1); the root's children carry tokens 1 then 2 and both uniforms are
    0.99, so both are rejected:
      - token 1: 0.99 * 0.5 >= 0.2. p_res = (p - q)+ = (.2, 0, 0, .1) / .3 = (2/3, 0, 0, 1/3);
        q_res = q without token 1 = (.1, 0, .3, .1) / .5 = (.2, 0, .6, .2);
      - token 2: 0.99 * 0.6 >= 0. p_res = (2/3 - .2, 0, 0, 1/3 - .2)+ = (7/15, 0, 0, 2/15),
        normalised (7/9, 0, 0, 2/9).
    The bonus is therefore token 0 for u_bonus < 7/9 and token 3 above."""
    p = np.array([0.3, 0.2, 0.3, 0.2])
    q = np.array([0.1, 0.5, 0.3, 0.1])
    parent = np.array([-1, -1], np.int32)
    token = np.array([1, 2], np.int32)
    u = np.array([0.99, 0.99])
    z = np.zeros((2, 4))
    for ub, want in ((0.0, 0), (0.7777, 0), (0.7778, 3), (0.999, 3)):
        path, y, _ = TA.accept_tree(p, q, z, z, parent, token, 0, 2, u, ub, TA.SAMPLE, 8)
        assert path == [] and y == want, (ub, y)
    # a rule that forgets to take the rejected token out of q_res subtracts q_res(2) = .3
    # and q_res(3) = .1 instead: p_res -> (17/24, 0, 0, 7/24), and u_bonus in
    # (17/24, 7/9) would give token 3
    for ub in (0.72, 0.75, 0.77):
        path, y, _ = TA.accept_tree(p, q, z, z, parent, token, 0, 2, u, ub, TA.SAMPLE, 8)
        assert y == 0, ub


def _closed_form_walk(p, q, toks, u, ub):
    """The residual in the closed form the acceptance kernel evaluates (kept here, in the
    test, to show it equals the oracle's step-by-step residual): after k rejections
    rp(y) = max(p(y) A - q(y) C, 0) unnormalised, with A <- A / Zp, C <- C / Zp + 1 / Zq,
    Zq <- Zq - q(x) per rejection of x and Zp = sum(rp). Returns (accepted sibling or -1,
    bonus, smallest relative margin)."""
    A, C, Zp, Zq = 1.0, 0.0, 1.0, 1.0
    rp = p.copy()
    fresh, margin = True, np.inf
    for c, x in enumerate(toks):
        rpx = max(p[x] * A - q[x] * C, 0.0)
        lhs, rhs = u[c] * q[x] * Zp, rpx * Zq
        margin = min(margin, TA._rel(lhs, rhs))
        if lhs < rhs:
            return c, None, margin
        A, C = A / Zp, C / Zp + 1.0 / Zq
        Zq -= q[x]
        rp = np.maximum(p * A - q * C, 0.0)
        Zp = float(rp.sum())
        fresh = False
    total = float(rp.sum()) if fresh else Zp
    cs = np.cumsum(rp)
    t = ub * total
    margin = min(margin, float(np.abs(cs - t).min()) / t)
    return -1, min(int(np.searchsorted(cs, t, side="right")), len(p) - 1), margin


def test_kernel_residual_form_equals_the_step_by_step_rule():
    """The acceptance kernel keeps the residual in a closed form instead of stepping it.
    In real arithmetic the two agree for siblings with distinct tokens (a clamp at 0 never
    releases, and a rejected token's residual is 0 already). Here both walk the same
    random sibling groups: every decision whose margin is clear agrees."""
    rng = np.random.default_rng(42)
    agree = 0
    for trial in range(400):
        V = int(rng.integers(3, 40))
        k = int(rng.integers(1, min(V, 6) + 1))
        p = rng.dirichlet(np.full(V, 0.5))
        q = rng.dirichlet(np.full(V, 0.5))
        toks = rng.choice(V, size=k, replace=False, p=q)
        u = rng.random(k)
        ub = float(rng.random())
        parent = np.full(k, -1, np.int32)
        z = np.zeros((k, V))
        path, y, m = TA.accept_tree(p, q, z, z, parent, toks, 0, k, u, ub, TA.SAMPLE, 8)
        c, yc, mc = _closed_form_walk(p, q, toks, u, ub)
        if min(m, mc) <= 1e-9:
            continue
        agree += 1
        assert (path[0] if path else -1) == c, trial
        if c < 0:
            assert y == yc, trial
    assert agree >= 390


def test_duplicate_siblings_are_a_bad_tree_under_sampling():
    """Two siblings with the same token are not a draft without replacement. The closed
    form would take q(x) out of Zq twice, the step-by-step rule subtracts q_res once more
    without removing anything: the section 9.1 guarantee holds for neither, so the batch
    call reports such a tree BAD_TOKEN under sampling. Greedy acceptance is well defined
    on it (the lowest-index child carrying the argmax) and accepts as usual."""
    V = 5
    parent = np.array([-1, -1, 0, 0, 0], np.int32)
    token = np.array([1, 3, 2, 4, 2], np.int32)       # nodes 2 and 4: same parent, token 2
    rng = np.random.default_rng(1)
    ctx = rng.dirichlet(np.ones(V), size=1).astype(np.float32)
    rows = rng.dirichlet(np.ones(V), size=5).astype(np.float32)
    offs = np.array([0, 5], np.int32)
    u = np.full(5, 0.5, np.float32)
    r = TA.accept_trees(ctx, ctx, rows, rows, parent, token, offs, u, np.full(1, 0.5, np.float32),
                        TA.SAMPLE, 4)
    assert r["status"].tolist() == [TA.TREE_BAD_TOKEN] and r["bonus"].tolist() == [-1]
    g = TA.accept_trees(ctx, None, rows, None, parent, token, offs, None, np.zeros(1),
                        TA.GREEDY, 4)
    assert g["status"].tolist() == [TA.TREE_OK]
    # the same token under different parents is fine
    token2 = np.array([1, 3, 2, 4, 1], np.int32)
    r2 = TA.accept_trees(ctx, ctx, rows, rows, parent, token2, offs, u, np.full(1, 0.5, np.float32),
                         TA.SAMPLE, 4)
    assert r2["status"].tolist() == [TA.TREE_OK]
    # and the closed form really does differ from the step-by-step rule on duplicates:
    # token 0 rejected twice, then token 1 (uniforms 0.99). Step by step, the second
    # rejection of token 0 leaves p_res = (0, 1, 0), q_res = (0, .5, .5), and token 1 is
    # accepted (0.99 * .5 < 1). The closed form takes q(0) out of Zq twice (Zq = -0.2),
    # and its test 0.99 * .2 * .1 < .1 * (-0.2) rejects token 1.
    p = np.array([0.1, 0.5, 0.4])
    q = np.array([0.6, 0.2, 0.2])
    z = np.zeros((3, 3))
    u3 = np.array([0.99, 0.99, 0.99])
    c_cf, _, _ = _closed_form_walk(p, q, [0, 0, 1], u3, 0.5)
    path, _, _ = TA.accept_tree(p, q, z, z, np.full(3, -1, np.int32), np.array([0, 0, 1], np.int32),
                                0, 3, u3, 0.5, TA.SAMPLE, 8)
    assert path == [2] and c_cf == -1
