"""Tree acceptance: which draft nodes the target model accepts, and its next token.

TEST INFRASTRUCTURE ONLY: the tests, the smoke entry and the benchmark's CPU-baseline leg
are its only callers; the GPU library never imports, loads or calls it.

It follows the LLM Primer chapter 9 walkthrough, section 9.1: the target scores every
drafted position in one pass, the longest prefix it agrees with is accepted, and at the
first disagreement the target's own choice is committed. With sampling, a token x drafted
from q is accepted with probability min(1, p(x) / q(x)); otherwise the token comes from
the normalised residual (p - q)+. That keeps the output distributed exactly as the
target's.

On a tree (the reading taken where the pages are silent):
  - the walk starts at the verified context and descends one accepted node at a time;
  - greedy (temperature 0): the target's choice at a node is its argmax (lowest token id
    on ties); the child carrying that token is accepted (the lowest-index one if several),
    and when no child carries it, that token is the next (bonus) token;
  - sampling: the children of the current node are tested in index order, each against
    the residual distributions the children rejected before it left. x is accepted when
    u * q_res(x) < p_res(x) (probability min(1, p_res(x) / q_res(x))). On a rejection,
    step by step:
        p_res <- max(p_res - q_res, 0), renormalised to sum 1;
        q_res[x] <- 0, q_res renormalised to sum 1
    (siblings are distinct tokens, drawn from q without replacement, so the rejected
    token leaves the draft distribution). When every child is rejected, or the node has
    none, the bonus token is drawn from p_res by inverse CDF with the tree's bonus
    uniform: the smallest y with sum_{y' <= y} p_res(y') > u * sum(p_res) (the last y if
    rounding leaves none). On a chain this is the section 9.1 rule exactly.
  - siblings with the same token are a malformed draft under sampling (the rule above
    assumes drafts without replacement): such a tree is reported BAD_TOKEN;
  - at most max_path nodes are accepted; the bonus is then drawn at the last one.

Arithmetic: fp64 numpy arrays, the residuals held normalised, one step per rejection in
the order above. Each call also returns the smallest relative decision margin it met
(acceptance tests and the bonus threshold), so that a test can tell a genuine mismatch
from a comparison that different rounding may flip.
"""
import numpy as np

GREEDY, SAMPLE = 0, 1
# per-tree status codes (same values as the C header's BOLE_TREE_*)
TREE_OK, TREE_BAD_SIZE, TREE_BAD_PARENT, TREE_BAD_TOKEN = 0, 1, 2, 4


def _rel(a, b):
    m = max(abs(a), abs(b))
    return abs(a - b) / m if m > 0 else 0.0


def _normalised(r):
    """r / sum(r); a vector with nothing left stays all zero."""
    s = float(r.sum())
    return r / s if s > 0 else np.zeros_like(r)


def accept_tree(p_ctx, q_ctx, p_node, q_node, parent, token, lo, n, u_node, u_bonus, mode,
                max_path):
    """One tree: rows lo .. lo + n - 1 of the packed node arrays. p_ctx, q_ctx are the
    rows at the verified context; p_node[lo + i], q_node[lo + i] the rows after node i.
    Returns (accepted tree-local indices, bonus token, smallest relative margin)."""
    kids = {-1: []}
    for i in range(n):
        kids.setdefault(i, [])
        kids.setdefault(int(parent[lo + i]), []).append(i)
    path, cur, margin = [], -1, np.inf
    while True:
        prow = np.asarray(p_ctx if cur < 0 else p_node[lo + cur], np.float64)
        room = len(path) < max_path
        if mode == GREEDY:
            y = int(np.argmax(prow))
            hit = [c for c in kids[cur] if int(token[lo + c]) == y]
            if hit and room:
                path.append(hit[0])
                cur = hit[0]
                continue
            return path, y, margin
        qrow = np.asarray(q_ctx if cur < 0 else q_node[lo + cur], np.float64)
        p_res = prow.copy()   # the target row as given at a fresh node
        q_res = qrow.copy()
        nxt = None
        for c in (kids[cur] if room else []):
            x = int(token[lo + c])
            lhs = float(u_node[lo + c]) * q_res[x]
            rhs = p_res[x]
            margin = min(margin, _rel(lhs, rhs))
            if lhs < rhs:
                nxt = c
                break
            p_res = _normalised(np.maximum(p_res - q_res, 0.0))
            q_res = q_res.copy()
            q_res[x] = 0.0
            q_res = _normalised(q_res)
        if nxt is not None:
            path.append(nxt)
            cur = nxt
            continue
        t = float(u_bonus) * float(p_res.sum())
        cs = np.cumsum(p_res)
        y = min(int(np.searchsorted(cs, t, side="right")), p_res.shape[0] - 1)
        if t > 0:
            margin = min(margin, float(np.abs(cs - t).min()) / t)
        return path, y, margin


def accept_trees(p_ctx, q_ctx, p_node, q_node, parent, token, node_offsets, u_node, u_bonus,
                 mode, max_path):
    """A packed batch. Returns dict of accepted_idx [B][max_path] (-1 padded),
    accepted_len [B], bonus [B], status [B], margin [B]. A tree whose offsets are out of
    order or outside [0, T] or hold more than 64 nodes gets BAD_SIZE, a parent outside
    [-1, i) BAD_PARENT, a token outside [0, V) BAD_TOKEN, and so do two siblings with the
    same token under sampling; such trees accept nothing and get bonus -1."""
    B = len(node_offsets) - 1
    T = len(parent)
    V = np.asarray(p_ctx).shape[-1]
    idx = np.full((B, max_path), -1, np.int32)
    ln = np.zeros(B, np.int32)
    bonus = np.full(B, -1, np.int32)
    status = np.zeros(B, np.int32)
    margin = np.full(B, np.inf)
    for b in range(B):
        lo, hi = int(node_offsets[b]), int(node_offsets[b + 1])
        if lo < 0 or hi < lo or hi > T or hi - lo > 64:
            status[b] = TREE_BAD_SIZE
            continue
        n = hi - lo
        if any(not (-1 <= int(parent[lo + i]) < i) for i in range(n)):
            status[b] = TREE_BAD_PARENT
            continue
        if any(not (0 <= int(token[lo + i]) < V) for i in range(n)):
            status[b] = TREE_BAD_TOKEN
            continue
        if mode == SAMPLE:
            pairs = [(int(parent[lo + i]), int(token[lo + i])) for i in range(n)]
            if len(set(pairs)) != n:
                status[b] = TREE_BAD_TOKEN
                continue
        path, y, m = accept_tree(p_ctx[b], q_ctx[b] if q_ctx is not None else None, p_node,
                                 q_node, parent, token, lo, n, u_node, u_bonus[b], mode,
                                 max_path)
        idx[b, :len(path)] = path
        ln[b] = len(path)
        bonus[b] = y
        margin[b] = m
    return {"accepted_idx": idx, "accepted_len": ln, "bonus": bonus, "status": status,
            "margin": margin}
