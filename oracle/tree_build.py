"""Best-first draft-tree construction and the hardware-aware budget controller.

TEST INFRASTRUCTURE ONLY: the tests, the smoke entry and the benchmark's CPU-baseline leg
are its only callers; the GPU library never imports, loads or calls it.

It follows the BASTION summary page ("Budget-Aware Speculative Decoding with
Tree-structured Block Diffusion Drafting"):
  - section 1, path scoring: a node i at depth d(i) whose path carries tokens
    x_i1 .. x_id has the path score rho(i) = prod_{k=1..d(i)} q_k(x_ik), where q_k is the
    drafter's position-wise marginal for position k;
  - section 2, acceptance surrogate and best-first expansion: the expected accepted length
    of a tree is estimated by A_hat(T) = sum_{i in T} rho(i), and the tree is grown by
    repeatedly inserting the valid node (one whose parent is already in the tree) with the
    highest rho;
  - section 3, online budget controller: the tree of N nodes is worth
    S(N) = A_hat(T_N) * L_AR / C(N), and the tree grows while S does not drop.

Precision. Every score (a product of fp32 probabilities) and every decision (which
candidate scores highest, whether S drops) is taken in fp32, in the order written here,
so that the kernels take the same decisions on the same values.
"""
import numpy as np

F32 = np.float32


def topk_desc(row, k):
    """The k largest entries of a 1-D array: (values fp32, indices int32), ordered by
    value descending, then index ascending (the rank order of the candidates)."""
    row = np.asarray(row, dtype=F32)
    k = min(int(k), row.shape[0])
    order = np.lexsort((np.arange(row.shape[0]), -row.astype(np.float64)))[:k]
    return row[order], order.astype(np.int32)


def best_first(top_vals, top_idx, n_max):
    """Best-first tree over per-depth candidate lists.

    top_vals[k][r], top_idx[k][r]: the r-th best token of position k + 1 (depth k + 1),
    as returned by topk_desc with at least min(n_max, V) entries per depth.

    Every node already in the tree (and the root context, whose children are the depth-1
    tokens) offers one candidate: its best child not yet inserted, i.e. the next rank at
    the next depth. The candidate's score is fp32(rho(parent) * q). Among all offers the
    highest score is inserted; ties go to the earlier source, the root context first,
    then tree nodes in insertion order. Node indices are insertion order, so a parent
    always precedes its children.

    Returns (parent, token, depth, rho) lists (parent -1 for a depth-1 node).
    """
    D = len(top_vals)
    parent, token, depth, rho = [], [], [], []
    next_rank = {-1: 0}
    for n in range(int(n_max)):
        best = None
        for s in [-1] + list(range(n)):
            d = 0 if s < 0 else depth[s]          # the offered child is at depth d + 1
            r = next_rank[s]
            if d >= D or r >= len(top_vals[d]):
                continue
            base = F32(1.0) if s < 0 else F32(rho[s])
            score = F32(base * F32(top_vals[d][r]))
            if best is None or score > best[0]:
                best = (score, s, d, r)
        if best is None:
            break
        score, s, d, r = best
        parent.append(s)
        token.append(int(top_idx[d][r]))
        depth.append(d + 1)
        rho.append(score)
        next_rank[s] = r + 1
        next_rank[n] = 0
    return parent, token, depth, rho


def controller(rho, cost, l_ar, fixed=False):
    """Tree size for one sequence from its scores in insertion order.

    A_hat(N) = rho_0 + ... + rho_{N-1}, summed in that order in fp32;
    S(N) = fp32(fp32(A_hat(N) * L_AR) / C(N)), C(N) = cost[N - 1].
    The tree grows from N = 1 while S(N + 1) >= S(N): the first N with S(N + 1) < S(N) is
    kept; else every built node. fixed=True keeps every built node (a fixed budget).
    Returns (N, S(N)); (0, 0) for an empty tree."""
    n_avail = len(rho)
    if n_avail == 0:
        return 0, F32(0.0)
    A = []
    acc = F32(0.0)
    for r in rho:
        acc = F32(acc + F32(r))
        A.append(acc)
    l_ar = F32(l_ar)

    def S(N):
        return F32(F32(A[N - 1] * l_ar) / F32(cost[N - 1]))

    n_keep = n_avail
    if not fixed:
        for N in range(1, n_avail):
            if S(N + 1) < S(N):
                n_keep = N
                break
    return n_keep, S(n_keep)


def build_trees(marginals, cost, l_ar, n_max, fixed=False):
    """Draft trees for a batch: marginals [B][D][V] (fp32 probabilities, position k of
    sequence b in row [b][k-1]), cost [>= n_max] (C(N) at index N - 1), L_AR.

    Returns a dict of numpy arrays: n_nodes [B], node_offsets [B + 1], and the packed
    per-node parent (tree-local), token, depth, rho, plus speedup [B] (S at the kept
    size)."""
    m = np.asarray(marginals, dtype=F32)
    B, D, V = m.shape
    K = min(int(n_max), V)
    out = {"n_nodes": [], "parent": [], "token": [], "depth": [], "rho": [], "speedup": []}
    for b in range(B):
        tops = [topk_desc(m[b, k], K) for k in range(D)]
        par, tok, dep, rho = best_first([t[0] for t in tops], [t[1] for t in tops], n_max)
        n_keep, s = controller(rho, cost, l_ar, fixed)
        out["n_nodes"].append(n_keep)
        out["parent"] += par[:n_keep]
        out["token"] += tok[:n_keep]
        out["depth"] += dep[:n_keep]
        out["rho"] += rho[:n_keep]
        out["speedup"].append(s)
    n_nodes = np.array(out["n_nodes"], dtype=np.int32)
    return {
        "n_nodes": n_nodes,
        "node_offsets": np.concatenate([[0], np.cumsum(n_nodes)]).astype(np.int32),
        "parent": np.array(out["parent"], dtype=np.int32),
        "token": np.array(out["token"], dtype=np.int32),
        "depth": np.array(out["depth"], dtype=np.int32),
        "rho": np.array(out["rho"], dtype=F32),
        "speedup": np.array(out["speedup"], dtype=F32),
    }
