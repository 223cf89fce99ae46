/*
 * bole_oracle.c - fp64 CPU oracle for Bole's tree verification and accepted-path commit.
 *
 * TEST INFRASTRUCTURE ONLY. The test-suite, the smoke entry and the benchmark's
 * CPU-baseline leg are the only callers. The GPU library neither links, loads nor
 * calls it, and the two share no code, header, table or helper.
 *
 * Source: "Bole: Efficient Tree Speculation for Hybrid-Attention Language Models",
 * as summarised on the llm-wiki page about Bole.
 *  - Section 1, "Tree-Structured Closed Form": the linear-attention recurrence
 *    h_{t+1} = S_t h_t + u_t, with a gating matrix S_t and an update term u_t per token.
 *  - Section 2, "Token-Level Factor Encoding": each node keeps only its own factor
 *    (S_i, u_i), and after verification only the accepted path's state is rebuilt.
 *  - "Comparison with prior approaches" table: the naive baseline walks the recurrence
 *    serially per branch and keeps one full state per draft node.
 *
 * Specialisation used here (the linear-recurrence layers of Mamba-2 / GLA / RWKV-6):
 *  - S_i = a_i * I (one scalar decay per token and head) or diag(g_i) (one decay per
 *    key channel, acting on the d_k rows);
 *  - u_i = k_i v_i^T;
 *  - a node's state is H_i = S_i H_parent(i) + k_i v_i^T, where H_parent = H_0 (the
 *    committed state) for a root, and its output is o_i = H_i^T q_i. The output is
 *    taken after the node's own update.
 *
 * This file evaluates all of that the naive way. For every node it copies H_0 and
 * applies, root first, the updates of every node on its root-to-node path. That costs
 * one full d_k x d_v state per node: slow and plainly correct. The parallel closed
 * form is what the GPU library computes, and this walk is what it is checked against.
 *
 * Layouts, all row-major and contiguous:
 *   H0    [B][H][d_k][d_v]
 *   q, k  [T][H][d_k]
 *   v     [T][H][d_v]
 *   gate  [T][H] (scalar) or [T][H][d_k] (vector)
 *   out   [T][H][d_v]
 * Tree b owns the packed nodes node_offsets[b] .. node_offsets[b+1]-1. parent[] holds
 * tree-local indices, with -1 meaning "child of the committed state".
 *
 * Per-tree status codes (the GPU library documents the same meanings):
 *   0 = ok;
 *   1 = bad size: the offsets are not ordered inside [0, T], or the tree has more
 *       than 64 nodes;
 *   2 = bad parent: some node i has parent[i] < -1 or parent[i] >= i;
 *   3 = bad path (commit only): the length is outside [0, max_path], or the path is
 *       not a chain that starts at a root.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_MAX_TREE 64

enum { OR_OK = 0, OR_BAD_SIZE = 1, OR_BAD_PARENT = 2, OR_BAD_PATH = 3 };

/* Number of OpenMP threads the parallel loops below use. */
int oracle_threads(void) { return omp_get_max_threads(); }

/* Threads for the parallel loops that follow (n >= 1); timing only, results do not depend on it. */
void oracle_set_threads(int n) { omp_set_num_threads(n > 0 ? n : 1); }

/* Structural check of tree b: size first, then every parent link. */
static int or_tree_check(int64_t b, const int32_t *node_offsets, int64_t total_nodes,
                         const int32_t *parent)
{
    int64_t lo = node_offsets[b], hi = node_offsets[b + 1];
    if (lo < 0 || hi < lo || hi > total_nodes || hi - lo > OR_MAX_TREE) return OR_BAD_SIZE;
    for (int64_t i = 0; i < hi - lo; ++i) {
        int32_t p = parent[lo + i];
        if (p < -1 || p >= i) return OR_BAD_PARENT;
    }
    return OR_OK;
}

/* Root-to-node path of tree-local node i (parents already checked): path[0] is the
 * root, path[d-1] == i. Returns d. */
static int or_path(const int32_t *par, int32_t i, int32_t *path)
{
    int32_t rev[OR_MAX_TREE];
    int d = 0;
    for (int32_t x = i; x >= 0; x = par[x]) rev[d++] = x;
    for (int m = 0; m < d; ++m) path[m] = rev[d - 1 - m];
    return d;
}

/* One recurrence step on an fp64 state: H <- S_j H + k_j v_j^T for packed node gj. */
static void or_step(double *H, int64_t gj, int64_t h, int64_t heads, int64_t d_k,
                    int64_t d_v, int vector_gate, const double *k, const double *v,
                    const double *gate)
{
    const double *kj = k + (gj * heads + h) * d_k;
    const double *vj = v + (gj * heads + h) * d_v;
    for (int64_t r = 0; r < d_k; ++r) {
        double s = vector_gate ? gate[(gj * heads + h) * d_k + r] : gate[gj * heads + h];
        for (int64_t c = 0; c < d_v; ++c) H[r * d_v + c] = s * H[r * d_v + c] + kj[r] * vj[c];
    }
}

/* Topology of every node: depth (= number of nodes on its root-to-node path) and the
 * ancestor-or-self bit mask (bit j set when tree-local node j lies on that path).
 * For a bad-parent tree, depth and mask are 0 for each of its nodes. For a bad-size
 * tree, nothing is written. Returns the number of bad trees. */
int oracle_topology(int64_t batch, int64_t total_nodes, const int32_t *node_offsets,
                    const int32_t *parent, int32_t *depth, uint64_t *mask, int32_t *status)
{
    int bad = 0;
    for (int64_t b = 0; b < batch; ++b) {
        int st = or_tree_check(b, node_offsets, total_nodes, parent);
        status[b] = st;
        if (st != OR_OK) ++bad;
        if (st == OR_BAD_SIZE) continue;
        int64_t lo = node_offsets[b], n = node_offsets[b + 1] - lo;
        for (int64_t i = 0; i < n; ++i) {
            depth[lo + i] = 0;
            mask[lo + i] = 0;
            if (st != OR_OK) continue;
            int32_t path[OR_MAX_TREE];
            int d = or_path(parent + lo, (int32_t)i, path);
            uint64_t m = 0;
            for (int t = 0; t < d; ++t) m |= (uint64_t)1 << path[t];
            depth[lo + i] = d;
            mask[lo + i] = m;
        }
    }
    return bad;
}

/* Cumulative log-decay of every node, summed root first along its path:
 * scalar: cumlog[T][H]; vector: cumlog[T][H][d_k]. Bad trees are skipped. */
int oracle_cumlog(int64_t batch, int64_t heads, int64_t d_k, int64_t total_nodes,
                  int vector_gate, const double *gate, const int32_t *parent,
                  const int32_t *node_offsets, double *cumlog)
{
    int64_t width = vector_gate ? d_k : 1;
    for (int64_t b = 0; b < batch; ++b) {
        if (or_tree_check(b, node_offsets, total_nodes, parent) != OR_OK) continue;
        int64_t lo = node_offsets[b], n = node_offsets[b + 1] - lo;
        for (int64_t i = 0; i < n; ++i) {
            int32_t path[OR_MAX_TREE];
            int d = or_path(parent + lo, (int32_t)i, path);
            for (int64_t h = 0; h < heads; ++h)
                for (int64_t c = 0; c < width; ++c) {
                    double acc = 0.0;
                    for (int t = 0; t < d; ++t)
                        acc += log(gate[((lo + path[t]) * heads + h) * width + c]);
                    cumlog[((lo + i) * heads + h) * width + c] = acc;
                }
        }
    }
    return 0;
}

/* Naive serial tree verification: out[i] = H_i^T q_i for every node, with H_i rebuilt
 * from H_0 by walking the node's path. Rows of a bad-parent tree are NaN. A bad-size
 * tree writes nothing. Returns the number of bad trees. */
int oracle_verify_serial(int64_t batch, int64_t heads, int64_t d_k, int64_t d_v,
                         int64_t total_nodes, int vector_gate, const double *H0,
                         const double *q, const double *k, const double *v,
                         const double *gate, const int32_t *parent,
                         const int32_t *node_offsets, double *out, int32_t *status)
{
    int bad = 0;
    for (int64_t b = 0; b < batch; ++b) {
        status[b] = or_tree_check(b, node_offsets, total_nodes, parent);
        if (status[b] != OR_OK) ++bad;
    }
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int64_t b = 0; b < batch; ++b) {
        for (int64_t h = 0; h < heads; ++h) {
            int st = status[b];
            if (st == OR_BAD_SIZE) continue;
            int64_t lo = node_offsets[b], n = node_offsets[b + 1] - lo;
            if (st != OR_OK) {
                for (int64_t i = 0; i < n; ++i)
                    for (int64_t c = 0; c < d_v; ++c)
                        out[((lo + i) * heads + h) * d_v + c] = NAN;
                continue;
            }
            double *H = (double *)malloc(sizeof(double) * d_k * d_v);
            const double *H0u = H0 + (b * heads + h) * d_k * d_v;
            for (int64_t i = 0; i < n; ++i) {
                int32_t path[OR_MAX_TREE];
                int d = or_path(parent + lo, (int32_t)i, path);
                memcpy(H, H0u, sizeof(double) * d_k * d_v);
                for (int t = 0; t < d; ++t)
                    or_step(H, lo + path[t], h, heads, d_k, d_v, vector_gate, k, v, gate);
                const double *qi = q + ((lo + i) * heads + h) * d_k;
                double *oi = out + ((lo + i) * heads + h) * d_v;
                for (int64_t c = 0; c < d_v; ++c) {
                    double acc = 0.0;
                    for (int64_t r = 0; r < d_k; ++r) acc += H[r * d_v + c] * qi[r];
                    oi[c] = acc;
                }
            }
            free(H);
        }
    }
    return bad;
}

/* Serial commit of the accepted path of every tree into H0, in place. The path of tree
 * b is accepted_idx[b][0 .. accepted_len[b]-1] (tree-local indices). It must start at
 * a root and follow parent links. H0 of tree b becomes the state after those tokens.
 * Length 0 leaves it unchanged. A tree with a nonzero status keeps its H0.
 * path_nodes (may be NULL), [B][max_path]: the packed indices node_offsets[b] + idx
 * that were applied, -1 elsewhere and for every bad tree. Returns the number of bad
 * trees. */
int oracle_commit_serial(int64_t batch, int64_t heads, int64_t d_k, int64_t d_v,
                         int64_t total_nodes, int vector_gate, double *H0, const double *k,
                         const double *v, const double *gate, const int32_t *parent,
                         const int32_t *node_offsets, const int32_t *accepted_idx,
                         const int32_t *accepted_len, int64_t max_path,
                         int32_t *path_nodes, int32_t *status)
{
    int bad = 0;
    for (int64_t b = 0; b < batch; ++b) {
        int st = or_tree_check(b, node_offsets, total_nodes, parent);
        if (st == OR_OK) {
            int64_t lo = node_offsets[b], n = node_offsets[b + 1] - lo;
            int32_t len = accepted_len[b];
            if (len < 0 || len > max_path) {
                st = OR_BAD_PATH;
            } else {
                int32_t prev = -1;
                for (int32_t m = 0; m < len; ++m) {
                    int32_t x = accepted_idx[b * max_path + m];
                    if (x < 0 || x >= n || parent[lo + x] != prev) { st = OR_BAD_PATH; break; }
                    prev = x;
                }
            }
        }
        status[b] = st;
        if (st != OR_OK) ++bad;
        if (path_nodes) {
            for (int64_t m = 0; m < max_path; ++m) {
                int ok = st == OR_OK && m < accepted_len[b];
                path_nodes[b * max_path + m] =
                    ok ? node_offsets[b] + accepted_idx[b * max_path + m] : -1;
            }
        }
    }
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int64_t b = 0; b < batch; ++b) {
        for (int64_t h = 0; h < heads; ++h) {
            if (status[b] != OR_OK) continue;
            double *Hu = H0 + (b * heads + h) * d_k * d_v;
            for (int32_t m = 0; m < accepted_len[b]; ++m) {
                int64_t gj = node_offsets[b] + accepted_idx[b * max_path + m];
                or_step(Hu, gj, h, heads, d_k, d_v, vector_gate, k, v, gate);
            }
        }
    }
    return bad;
}
