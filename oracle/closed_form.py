"""fp64 closed-form tree verification and path restore (test-only).

TEST INFRASTRUCTURE ONLY. This module states, as dense fp64 matrix algebra, the closed
form that Bole's summary page derives in section 1 ("Tree-Structured Closed Form"):
unrolling h_{t+1} = S_t h_t + u_t along a root-to-node chain gives the state as a
product of gating factors applied to h_0, plus the sum of each earlier update decayed
by the factors that follow it. Section 2 ("Token-Level Factor Encoding") restores the
accepted path's state from its factors in the same way.

With A_j = a_j I (scalar gate) or diag(g_j) (vector gate), and path(i) the chain of
nodes from a root down to i (i included):
    H_i = (prod_{m in path(i)} A_m) H_0 + sum_{j in path(i)} (prod_{m in path(i), m after j} A_m) k_j v_j^T
    o_i = H_i^T q_i
For a scalar gate this is o_i = D_i H_0^T q_i + sum_{j in path(i)} (D_i / D_j)(q_i . k_j) v_j,
with D_x the product of a over path(x).

The ancestor relation is built here as the transitive closure of the parent adjacency,
by repeated boolean squaring. That is deliberately unlike the serial per-node walk in
``bole_oracle.c``, so that the two fp64 evaluations check each other.
"""
import numpy as np


def ancestor_matrix(parent_local) -> np.ndarray:
    """M[i, j] = True iff tree-local node j lies on the root-to-i path (i included)."""
    p = np.asarray(parent_local, dtype=np.int64)
    n = p.shape[0]
    M = np.eye(n, dtype=bool)
    for i in range(n):
        if p[i] >= 0:
            M[i, p[i]] = True
    # closure: M <- M or M.M until stable (path lengths double each round)
    while True:
        M2 = M | ((M.astype(np.int64) @ M.astype(np.int64)) > 0)
        if np.array_equal(M2, M):
            return M
        M = M2


def verify_closed_form(H0, q, k, v, gate, parent, node_offsets, vector_gate):
    """All node outputs of every tree, [T, H, d_v] fp64, by the dense closed form.
    Inputs are fp64 arrays in the library layouts (H0 [B,H,dk,dv], q/k [T,H,dk],
    v [T,H,dv], gate [T,H] or [T,H,dk]). Trees must be valid."""
    B, Hn, d_k, d_v = H0.shape
    T = q.shape[0]
    out = np.full((T, Hn, d_v), np.nan)
    for b in range(B):
        lo, hi = int(node_offsets[b]), int(node_offsets[b + 1])
        if hi == lo:
            continue
        M = ancestor_matrix(parent[lo:hi]).astype(np.float64)
        for h in range(Hn):
            Q, K, V = q[lo:hi, h], k[lo:hi, h], v[lo:hi, h]
            if vector_gate:
                G = np.exp(M @ np.log(gate[lo:hi, h]))          # [n, d_k] cumulative decay
                Qt = G * Q
                S = Qt @ (K / G).T                              # S_ij = sum_c q_i k_j G_i/G_j
                out[lo:hi, h] = Qt @ H0[b, h] + (S * M) @ V
            else:
                D = np.exp(M @ np.log(gate[lo:hi, h]))          # [n]
                W = (Q @ K.T) * (D[:, None] / D[None, :]) * M
                out[lo:hi, h] = D[:, None] * (Q @ H0[b, h]) + W @ V
    return out


def restore_closed_form(H0, k, v, gate, node_offsets, accepted_idx, accepted_len, vector_gate):
    """Committed state after each tree's accepted path, fp64, by the closed form
    H' = (prod A) H_0 + K_p^T diag-decay V_p (paths must be valid)."""
    H = np.array(H0, dtype=np.float64, copy=True)
    B, Hn, d_k, d_v = H.shape
    for b in range(B):
        L = int(accepted_len[b])
        if L == 0:
            continue
        idx = int(node_offsets[b]) + np.asarray(accepted_idx[b][:L], dtype=np.int64)
        for h in range(Hn):
            Kp, Vp = k[idx, h], v[idx, h]
            if vector_gate:
                lg = np.log(gate[idx, h])                        # [L, d_k]
                tail = np.cumsum(lg[::-1], axis=0)[::-1]         # sum over m' >= m
                after = np.exp(tail - lg)                        # product over m' > m
                total = np.exp(tail[0])
                H[b, h] = total[:, None] * H[b, h] + (Kp * after).T @ Vp
            else:
                lg = np.log(gate[idx, h])                        # [L]
                tail = np.cumsum(lg[::-1])[::-1]
                after = np.exp(tail - lg)
                H[b, h] = np.exp(tail[0]) * H[b, h] + (Kp * after[:, None]).T @ Vp
    return H
