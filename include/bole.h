/*
 * bole.h - C ABI of the MI355X (gfx950) library for Bole-style tree verification of
 * linear-recurrence layers, and for the commit of the accepted path.
 *
 * Method: "Bole: Efficient Tree Speculation for Hybrid-Attention Language Models", as
 * summarised on the llm-wiki page about Bole.
 *  - Section 1, "Tree-Structured Closed Form": the per-token recurrence
 *    h_{t+1} = S_t h_t + u_t unrolls into a chain of factor products. Every draft node
 *    can therefore be verified in parallel, with no serial walk down the branches.
 *  - Section 2, "Token-Level Factor Encoding": each draft node stores only its own
 *    token factor, and after verification only the accepted path's state is rebuilt.
 *
 * Here, for the Mamba-2 / GLA / RWKV-6 family, a draft node i carries:
 *  - a gate: a scalar decay a_i per head (S_i = a_i I), or one decay per key channel
 *    g_i (S_i = diag(g_i), scaling the d_k rows of the state);
 *  - a rank-one update u_i = k_i v_i^T;
 *  - a query q_i.
 * Its state is H_i = S_i H_parent(i) + k_i v_i^T. A node whose parent is -1 hangs
 * directly off the committed state H_0. Its output, taken after its own update, is
 *     o_i = H_i^T q_i = D_i (H_0^T q_i) + sum_{j on path(i)} D_{j->i} (q_i . k_j) v_j
 * for a scalar gate, where D_i is the product of the gates on the root-to-i path and
 * D_{j->i} the product over the nodes after j on that path (D_{i->i} = 1). For a vector
 * gate the same holds channel by channel:
 *     o_i = H_0^T (G_i * q_i) + sum_j (sum_c q_i[c] k_j[c] G_i[c] / G_j[c]) v_j.
 *
 * Memory layouts. Everything is row-major, contiguous, and in device memory unless
 * stated otherwise:
 *   H0    float [B][H][d_k][d_v]   committed state, one matrix per (sequence, head)
 *   q, k  [T][H][d_k]              factor_dtype (bf16 or fp32)
 *   v     [T][H][d_v]              factor_dtype
 *   gate  float [T][H] (BOLE_GATE_SCALAR) or [T][H][d_k] (BOLE_GATE_VECTOR).
 *         It holds the decay itself: finite and > 0, typically in (0, 1].
 *   out   float [T][H][d_v]
 *   parent       int32 [T]      tree-local parent index, -1 for a root. parent[i] < i
 *                               is required (topological order). Forests are allowed.
 *   node_offsets int32 [B + 1]  tree b owns packed rows node_offsets[b] ..
 *                               node_offsets[b+1]-1, at most 64 of them.
 *   accepted_idx int32 [B][max_path]  tree-local accepted path, root first
 *   accepted_len int32 [B]
 * Rows that belong to no tree are neither read nor written.
 *
 * Ownership. The caller owns every buffer. The library allocates nothing, keeps no
 * pointer after a call returns, and verify, commit and prepare need no workspace
 * (bole_workspace_bytes returns 0; the tree builder alone takes one). Every call except
 * bole_read_status is asynchronous on the given stream and does not synchronise. Calls
 * are reentrant across streams.
 *
 * Errors.
 *  - Problems visible on the host (null pointers, sizes out of range, unsupported
 *    combinations) are reported by the return value before anything is launched.
 *  - Problems in tree data are only visible on the device. They are reported per tree
 *    in the optional tree_status[B] output, as BOLE_TREE_* codes:
 *      - for a tree with a bad size, nothing is written;
 *      - verify fills the rows of a bad-parent tree with NaN;
 *      - commit leaves the state of any bad tree untouched.
 *    bole_read_status copies the array to the host after the stream's work and returns
 *    BOLE_ERR_BAD_TREE when any tree is bad.
 *  - Gates are not checked unless BOLE_FLAG_VALIDATE_GATES is set: a gate outside its
 *    domain (finite and > 0) then makes the tree BOLE_TREE_BAD_GATE, handled like a
 *    bad-parent tree (NaN rows from verify, untouched state from commit).
 */
#ifndef BOLE_H
#define BOLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BOLE_API __attribute__((visibility("default")))

/* Host-side result of every call. */
typedef enum {
    BOLE_OK = 0,
    BOLE_ERR_INVALID_VALUE = 1, /* null pointer, negative size, bad enum value */
    BOLE_ERR_UNSUPPORTED = 2,   /* valid request outside what the kernels cover */
    BOLE_ERR_HIP = 3,           /* a HIP launch, copy or synchronisation reported an error */
    BOLE_ERR_BAD_TREE = 4       /* bole_read_status: at least one tree is not BOLE_TREE_OK */
} bole_status_t;

/* Per-tree device-side status written to tree_status[b]. */
enum {
    BOLE_TREE_OK = 0,
    BOLE_TREE_BAD_SIZE = 1,   /* offsets unordered, outside [0, T], or more than 64 nodes
                                 (32 under BOLE_FLAG_TREES_LE_32) */
    BOLE_TREE_BAD_PARENT = 2, /* some node i has parent[i] < -1 or parent[i] >= i */
    BOLE_TREE_BAD_PATH = 3,   /* commit: length outside [0, max_path], an index outside
                                 the tree, or not a chain that starts at a root */
    BOLE_TREE_BAD_TOKEN = 4,  /* accept: a node's token outside [0, vocab), or (sampling)
                                 two siblings carrying the same token */
    BOLE_TREE_BAD_GATE = 5    /* under BOLE_FLAG_VALIDATE_GATES: a gate of one of the tree's
                                 nodes (any layer, head or channel) is not finite and > 0 */
};

typedef enum { BOLE_DTYPE_BF16 = 0, BOLE_DTYPE_F32 = 1 } bole_dtype_t;
typedef enum { BOLE_GATE_SCALAR = 0, BOLE_GATE_VECTOR = 1 } bole_gate_kind_t;

/* Flags (bole_dims_t.flags). */
enum {
    BOLE_FLAG_FORCE_GENERIC = 1, /* use the plain vector-ALU kernels even where the
                                    matrix-core kernels apply (testing, odd shapes) */
    BOLE_FLAG_TREES_LE_32 = 2,   /* the caller's tree budget is at most 32 nodes: only the
                                    kernels for such trees are launched, and a tree with
                                    more nodes is reported BOLE_TREE_BAD_SIZE (verify and
                                    commit alike) and left untouched */
    BOLE_FLAG_VALIDATE_GATES = 4 /* check every gate of every tree's nodes (in every layer
                                    of the call) against its domain, finite and > 0, on the
                                    device. A structurally valid tree with a bad gate gets
                                    BOLE_TREE_BAD_GATE: verify writes NaN over its rows in
                                    every layer, commit keeps its state in every layer.
                                    tree_status is then required (NULL gives
                                    BOLE_ERR_INVALID_VALUE). It costs one extra read of the
                                    gates (verify: after the verify kernels, plus a pass
                                    that rewrites the rows of bad trees; commit: before the
                                    commit kernels); the lazy calls run as commit then
                                    verify under it. Without the flag a bad gate changes
                                    only the values of its own tree's outputs and state. */
};

/* Same type as hipStream_t; NULL is the default stream. */
typedef struct ihipStream_t *bole_stream_t;

typedef struct {
    int32_t batch;        /* B >= 0 trees (one per sequence) */
    int32_t heads;        /* H >= 1 */
    int32_t d_k;          /* key width = state rows, 1..256 */
    int32_t d_v;          /* value width = state columns, 1..256 */
    int32_t total_nodes;  /* T >= 0, rows of the packed node arrays */
    int32_t max_path;     /* commit: row stride of accepted_idx, 0..64 */
    int32_t factor_dtype; /* bole_dtype_t of q, k, v */
    int32_t gate_kind;    /* bole_gate_kind_t */
    int32_t flags;        /* BOLE_FLAG_* */
} bole_dims_t;

/* Per-node factors that a commit gathers along the accepted path (section 2 of the
 * Bole summary: the factors (S_i, u_i) are all that is kept per node). */
typedef struct {
    const void *k;                /* [T][H][d_k] factor_dtype */
    const void *v;                /* [T][H][d_v] factor_dtype */
    const float *gate;            /* [T][H] or [T][H][d_k] */
    const int32_t *parent;        /* [T] */
    const int32_t *node_offsets;  /* [B + 1] */
} bole_factors_t;

/* One layer of a stack of linear-recurrence layers. The layers of a stack see the same
 * draft tokens, so they verify the same trees and commit the same accepted paths; only
 * each layer's state and per-node factors are its own. Every pointer follows the layouts
 * above, with the same dims for every layer. A host struct of device pointers. */
typedef struct {
    float *H0;              /* [B][H][d_k][d_v] this layer's committed state */
    const void *q;          /* [T][H][d_k] this step's factors */
    const void *k;          /* [T][H][d_k] */
    const void *v;          /* [T][H][d_v] */
    const float *gate;      /* [T][H] or [T][H][d_k] */
    float *out;             /* [T][H][d_v] verify output; unused by commit */
    const void *prev_k;     /* lazy commit only: the previous step's k, v and gate, */
    const void *prev_v;     /* laid out by that step's tree; NULL elsewhere */
    const float *prev_gate;
} bole_layer_t;

/* Maximum number of nodes in one tree (one 64-lane wavefront, one 64-bit mask). */
BOLE_API int32_t bole_max_tree_nodes(void);

/* Human-readable name of a status value (static string, never NULL). */
BOLE_API const char *bole_status_string(bole_status_t status);

/* Host-only check of a dims descriptor, the same check every entry point runs first.
 * `op` is 0 for verify, 1 for commit, 2 for prepare. Touches no device. */
BOLE_API bole_status_t bole_check_dims(const bole_dims_t *dims, int32_t op);

/* Scratch bytes that bole_tree_verify, bole_commit_path, their lazy and layer-stack forms
 * and bole_tree_prepare need: always 0. Their kernels keep every intermediate (topology,
 * cumulative decay, pair weights, partial sums) in registers and LDS, and per-tree
 * statuses go to the caller's tree_status array. dims may be NULL. */
BOLE_API size_t bole_workspace_bytes(const bole_dims_t *dims);

/*
 * Reads the per-tree statuses of earlier calls: a copy of tree_status[0 .. batch-1]
 * (device int32, as written by any entry point) ordered after the work already on
 * `stream`, then a synchronisation of `stream`. This is the one call that blocks the
 * host. host_status (host int32[batch], may be NULL) receives the values. Returns
 * BOLE_ERR_BAD_TREE if any value is not BOLE_TREE_OK, BOLE_OK if all are,
 * BOLE_ERR_INVALID_VALUE for batch < 0 or a NULL tree_status with batch > 0, and
 * BOLE_ERR_HIP if the copy or the synchronisation fails. Nothing is allocated: without
 * host_status the values pass through a buffer on the stack, 256 at a time.
 */
BOLE_API bole_status_t bole_read_status(const int32_t *tree_status, int32_t batch,
                                        int32_t *host_status, bole_stream_t stream);

/*
 * Tree verification: the closed form of the Bole summary page, section 1
 * ("Tree-Structured Closed Form").
 * Writes out[i] = H_i^T q_i for every node of every tree, all nodes in parallel.
 * H0 is read once per (sequence, head) and never written. No per-node state is ever
 * materialised: only the per-node factors are read.
 * out must not alias any input.
 * tree_status (device int32[B], may be NULL) receives one BOLE_TREE_* code per tree.
 * Returns BOLE_ERR_INVALID_VALUE or BOLE_ERR_UNSUPPORTED without launching anything.
 */
BOLE_API bole_status_t bole_tree_verify(const float *H0, const void *q, const void *k, const void *v,
                               const float *gate, const int32_t *parent,
                               const int32_t *node_offsets, float *out,
                               const bole_dims_t *dims, int32_t *tree_status,
                               bole_stream_t stream);

/*
 * Lazy commit: the previous step's accepted-path commit folded into this step's verify,
 * so that one pass over H0 serves both. The restore of the Bole summary page, section 2
 * ("Token-Level Factor Encoding": after verification only the accepted path's state is
 * rebuilt), followed by the closed form of section 1; the pages do not say when the
 * restore runs, and nothing reads the committed state before the next step's verify. The accepted path of a step is known only after
 * that step's verify, so its commit can ride on the next step's verify; H0 is then read
 * once and written once per step instead of read twice and written once.
 * The result is that of
 *     bole_commit_path(H0, prev, prev_accepted_idx, prev_accepted_len, prev_dims,
 *                      prev_path_nodes, prev_tree_status, stream);
 *     bole_tree_verify(H0, q, k, v, gate, parent, node_offsets, out, dims, tree_status,
 *                      stream);
 * with the same statuses and path rows, and states and outputs equal to fp32 rounding
 * (the same products and sums, which the two forms' kernels may contract differently).
 * Every argument follows those two calls. prev_dims describes the previous step
 * (its total_nodes, max_path and flags); batch, heads, d_k, d_v, factor_dtype and
 * gate_kind must equal those of dims (else BOLE_ERR_INVALID_VALUE). On exit H0 holds
 * the state after the previous step's accepted tokens: the state the next call, or a
 * final bole_commit_path of the last step, starts from. The one-pass kernels cover bf16
 * factors with scalar or per-channel gates, d_k 64 or 128, d_v 32..256 and 16-byte
 * aligned rows, every tree size up to 64 nodes; any other shape, and a call under
 * BOLE_FLAG_VALIDATE_GATES, runs as the two calls above.
 */
BOLE_API bole_status_t bole_tree_verify_lazy_commit(
    float *H0, const bole_factors_t *prev, const int32_t *prev_accepted_idx,
    const int32_t *prev_accepted_len, const bole_dims_t *prev_dims, int32_t *prev_path_nodes,
    int32_t *prev_tree_status, const void *q, const void *k, const void *v, const float *gate,
    const int32_t *parent, const int32_t *node_offsets, float *out, const bole_dims_t *dims,
    int32_t *tree_status, bole_stream_t stream);

/*
 * Layer stacks: the calls above for num_layers >= 1 layers that share their trees (and
 * paths), in as few launches as the kernels allow. The Bole summary page applies the
 * closed form (section 1) and the restore (section 2) to every linear-recurrence layer of
 * a hybrid model; its draft tokens, and so its trees and accepted paths, are the same in
 * every layer. The matrix-core kernels take up to
 * 16 layers per launch (blockIdx.y = layer), so that the workgroups of one layer's tail
 * overlap the next layer's, instead of one launch, ramp and drain per layer. `layers` is
 * a host array of num_layers entries. Each call's result is exactly that of the
 * single-layer call on every layer in turn:
 *  - bole_tree_verify_layers: bole_tree_verify(layer.H0, layer.q, layer.k, layer.v,
 *    layer.gate, parent, node_offsets, layer.out, dims, tree_status, stream);
 *  - bole_commit_path_layers: bole_commit_path(layer.H0, {layer.k, layer.v, layer.gate,
 *    parent, node_offsets}, accepted_idx, accepted_len, dims, path_nodes, tree_status,
 *    stream);
 *  - bole_tree_verify_lazy_commit_layers: bole_tree_verify_lazy_commit(layer.H0,
 *    {layer.prev_k, layer.prev_v, layer.prev_gate, prev_parent, prev_node_offsets},
 *    prev_accepted_idx, prev_accepted_len, prev_dims, prev_path_nodes, prev_tree_status,
 *    layer.q, layer.k, layer.v, layer.gate, parent, node_offsets, layer.out, dims,
 *    tree_status, stream).
 * The per-tree outputs (tree_status, path_nodes, ...) depend on the trees alone and are
 * written once. Layers must not overlap in H0 (commit, lazy commit) or out (verify,
 * lazy commit); two layers with the same H0 or out pointer, num_layers < 1 or a NULL
 * layers array give BOLE_ERR_INVALID_VALUE.
 */
BOLE_API bole_status_t bole_tree_verify_layers(const bole_layer_t *layers, int32_t num_layers,
                               const int32_t *parent, const int32_t *node_offsets,
                               const bole_dims_t *dims, int32_t *tree_status,
                               bole_stream_t stream);

BOLE_API bole_status_t bole_commit_path_layers(const bole_layer_t *layers, int32_t num_layers,
                               const int32_t *parent, const int32_t *node_offsets,
                               const int32_t *accepted_idx, const int32_t *accepted_len,
                               const bole_dims_t *dims, int32_t *path_nodes,
                               int32_t *tree_status, bole_stream_t stream);

BOLE_API bole_status_t bole_tree_verify_lazy_commit_layers(
    const bole_layer_t *layers, int32_t num_layers, const int32_t *prev_parent,
    const int32_t *prev_node_offsets, const int32_t *prev_accepted_idx,
    const int32_t *prev_accepted_len, const bole_dims_t *prev_dims, int32_t *prev_path_nodes,
    int32_t *prev_tree_status, const int32_t *parent, const int32_t *node_offsets,
    const bole_dims_t *dims, int32_t *tree_status, bole_stream_t stream);

/*
 * Baseline: the naive serial walk that the closed form replaces: the one-state-per-node
 * approach of the Bole summary page's comparison with prior approaches (a full recurrent
 * state kept for every draft node, each branch walked serially; section 1 states the
 * recurrence it walks). Every node's state is materialised, in tree order:
 *     H_i = S_i H_parent(i) + k_i v_i^T   (H_parent = H0 for a root),   out[i] = H_i^T q_i.
 * states (device float [T][H][d_k][d_v], caller-owned: T * H * d_k * d_v floats)
 * receives every H_i; this is the transient memory the closed form avoids. Inputs,
 * outputs, tree_status and errors follow bole_tree_verify (bad-parent trees get NaN rows
 * and no states; bad-size trees are not touched). It exists to measure the closed form
 * against and is not a fast path.
 */
BOLE_API bole_status_t bole_tree_verify_naive(const float *H0, const void *q, const void *k,
                               const void *v, const float *gate, const int32_t *parent,
                               const int32_t *node_offsets, float *out, float *states,
                               const bole_dims_t *dims, int32_t *tree_status,
                               bole_stream_t stream);

/*
 * Accepted-path commit: the restore step of the Bole summary page, section 2
 * ("Token-Level Factor Encoding").
 * For each tree b with accepted_len[b] = L > 0, and path p_1..p_L
 * (= accepted_idx[b][0..L-1]):
 *     H0[b,h] <- S_{p_L}...S_{p_1} H0[b,h] + sum_m (S_{p_L}...S_{p_{m+1}}) k_{p_m} v_{p_m}^T
 * This is done in place, for every head. The result is the state after the accepted
 * tokens. A length of 0 leaves H0 untouched.
 * `factors` is a host struct of device pointers. accepted_idx and accepted_len are
 * device arrays.
 * path_nodes (device int32[B][max_path], may be NULL) receives the packed row of each
 * applied node (node_offsets[b] + accepted_idx[b][m]), and -1 elsewhere and for bad
 * trees.
 * tree_status (device int32[B], may be NULL) receives BOLE_TREE_* codes.
 * Must be stream-ordered after any verify that reads the same H0.
 */
BOLE_API bole_status_t bole_commit_path(float *H0, const bole_factors_t *factors,
                               const int32_t *accepted_idx, const int32_t *accepted_len,
                               const bole_dims_t *dims, int32_t *path_nodes,
                               int32_t *tree_status, bole_stream_t stream);

/*
 * Tree topology preprocessor: the same per-tree pass that verify and commit run
 * internally, exported on its own. It computes the two quantities the closed form of the
 * Bole summary page, section 1, needs per node: which nodes lie on its root-to-node path
 * (the ancestors j of the sum over the path) and the product of the gates along that
 * path (D_i, kept as a sum of logarithms).
 * Per node:
 *   depth  (int32 [T])  number of nodes on the root-to-node path;
 *   mask   (uint64 [T]) bit j set when tree-local node j is on that path;
 *   cumlog (float [T][H], or [T][H][d_k] for vector gates) sum of log(gate) over the
 *          path, root first.
 * Any output pointer may be NULL to skip that output. gate may be NULL when cumlog is
 * NULL.
 * For a bad-parent tree, depth, mask and cumlog are written as 0. For a bad-size tree,
 * nothing is written.
 */
BOLE_API bole_status_t bole_tree_prepare(const int32_t *parent, const int32_t *node_offsets,
                                const float *gate, const bole_dims_t *dims, int32_t *depth,
                                uint64_t *mask, float *cumlog, int32_t *tree_status,
                                bole_stream_t stream);

/*
 * Draft-tree construction and budget control: the BASTION summary page, sections 1-3.
 *  - Path score (section 1): node i at depth d(i) with path tokens x_i1..x_id scores
 *    rho(i) = prod_k q_k(x_ik), q_k being the drafter's position-wise marginal of
 *    position k.
 *  - Best-first expansion (section 2): the tree grows by repeatedly inserting the valid
 *    node (its parent already in the tree; depth-1 nodes hang off the verified context)
 *    with the highest rho. Each product is fp32(rho(parent) * q); ties go to the earlier
 *    source (the context first, then tree nodes in insertion order), and among one
 *    parent's children to the lower token id.
 *  - Budget controller (section 3): with A_hat(N) the fp32 sum of the first N scores in
 *    insertion order, S(N) = fp32(fp32(A_hat(N) * l_ar) / cost[N - 1]). The tree grows from
 *    N = 1 and keeps the first N with S(N + 1) < S(N), else all n_max nodes (or all
 *    nodes that exist). BOLE_BUILD_FIXED_BUDGET keeps n_max nodes without the test.
 *
 * Inputs:
 *   marginals float [B][depth][vocab]  q_k for positions k = 1..depth (probabilities,
 *                                      finite and >= 0; NaN is not allowed)
 *   cost      float [n_max]            cost[N - 1] = C(N), the caller's estimate of one
 *                                      step's time with an N-node tree (draft + verify),
 *                                      > 0; may be NULL with BOLE_BUILD_FIXED_BUDGET and
 *                                      speedup NULL
 *   l_ar                               L_AR, the autoregressive time per token, > 0 (same
 *                                      unit as cost)
 *   workspace                          device scratch of at least
 *                                      bole_build_tree_workspace_size(dims) bytes,
 *                                      16-byte aligned, owned by the caller; contents on
 *                                      entry do not matter
 * Outputs (device):
 *   node_offsets int32 [B + 1]   packed layout of the kept trees (as bole_tree_verify
 *                                takes it)
 *   parent int32 [B * n_max]     tree-local parent (-1 for depth 1), insertion order, so
 *                                parent[i] < i; rows past node_offsets[B] are not written
 *   token  int32 [B * n_max]     vocabulary index of each node
 *   rho    float [B * n_max]     path score of each node (may be NULL)
 *   speedup float [B]            S(N) at the kept size (may be NULL)
 * Host errors (BOLE_ERR_INVALID_VALUE / BOLE_ERR_UNSUPPORTED) are returned before any
 * launch: depth outside 1..32, n_max outside 1..64, vocab < 1, a short or misaligned
 * workspace, missing pointers, l_ar not > 0.
 */
enum { BOLE_BUILD_FIXED_BUDGET = 1 };

typedef struct {
    int32_t batch;  /* B >= 0 sequences */
    int32_t depth;  /* drafted positions per sequence, 1..32 */
    int32_t vocab;  /* vocabulary size, >= 1 */
    int32_t n_max;  /* tree budget cap, 1..64 */
    int32_t flags;  /* BOLE_BUILD_* */
} bole_build_dims_t;

/* Workspace bytes bole_build_tree needs for these dims (0 for invalid dims). */
BOLE_API size_t bole_build_tree_workspace_size(const bole_build_dims_t *dims);

BOLE_API bole_status_t bole_build_tree(const float *marginals, const float *cost, float l_ar,
                               void *workspace, size_t workspace_bytes,
                               const bole_build_dims_t *dims, int32_t *node_offsets,
                               int32_t *parent, int32_t *token, float *rho, float *speedup,
                               bole_stream_t stream);

/*
 * bole_build_tree without a workspace argument, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc). The three launches use a scratch array that the library holds on each GPU
 * (BOLE_BUILD_NOALLOC_MAX_BYTES, allocated by the code-object loader, kept until the
 * process ends) instead of the caller's workspace; nothing is allocated or freed here.
 * Dims whose bole_build_tree_workspace_size exceeds BOLE_BUILD_NOALLOC_MAX_BYTES give
 * BOLE_ERR_UNSUPPORTED before anything is launched (64 sequences x 8 positions x 128,256
 * tokens need about 1.1 MB). The stream must belong to the current device. Every call on
 * one GPU shares that GPU's array: calls that overlap on one GPU (other streams, other
 * threads) race, so serialise them. Nothing in the array needs clearing between calls.
 * Every other argument, output and error is that of bole_build_tree, and so are the
 * results, bit for bit.
 */
#define BOLE_BUILD_NOALLOC_MAX_BYTES ((size_t)4 << 20)
BOLE_API bole_status_t bole_build_tree_noalloc(const float *marginals, const float *cost,
                                               float l_ar, const bole_build_dims_t *dims,
                                               int32_t *node_offsets, int32_t *parent,
                                               int32_t *token, float *rho, float *speedup,
                                               bole_stream_t stream);

/*
 * Tree acceptance: the LLM Primer chapter 9 walkthrough, section 9.1. The target model
 * scores every drafted node in one pass; the walk from the verified context accepts the
 * longest path the target agrees with, and the target's own next token at the first
 * disagreement (the bonus token) is returned beside it.
 *  - BOLE_ACCEPT_GREEDY: at each node the target's choice is the argmax of its row
 *    (lowest token id on ties). The child carrying it is accepted (the lowest-index
 *    child if several); when none does, that token is the bonus.
 *  - BOLE_ACCEPT_SAMPLE: a drafted token x is accepted with probability
 *    min(1, p(x) / q(x)), else the bonus is drawn from the normalised residual (p - q)+,
 *    which keeps the output distributed as the target's. Siblings (distinct tokens,
 *    drafted without replacement; two siblings with one token make the tree
 *    BOLE_TREE_BAD_TOKEN) are tested in index order, each against the residuals
 *    the rejected ones before it left: p_res <- (p_res - q_res)+ renormalised, and the
 *    rejected token leaves q_res, renormalised. x is accepted when
 *    u_node[x's node] * q_res(x) < p_res(x). The bonus is the smallest y whose
 *    cumulative p_res exceeds u_bonus[b] (inverse CDF). Residuals are fp64; draws that
 *    fall within rounding of a boundary may differ from a different summation order.
 * At most max_path nodes are accepted; the bonus is then taken at the last of them.
 *
 * Inputs (device, fp32 probability rows, each finite, >= 0 and summing to 1):
 *   p_ctx [B][V], q_ctx [B][V]    target / draft distribution at the verified context
 *   p_node [T][V], q_node [T][V]  the same after each draft node (q: the distribution
 *                                 its children were drafted from)
 *   parent [T], token [T], node_offsets [B + 1]   the packed trees (as verify takes them)
 *   u_node [T], u_bonus [B]       uniforms in [0, 1) (sampling)
 *   q_ctx, q_node, u_node, u_bonus may be NULL for greedy. No workspace: the residuals
 *   are recomputed from the rows (same fp64 operations, same order) instead of stored.
 * Outputs (device): accepted_idx [B][max_path] (tree-local, root first, -1 after the
 * path), accepted_len [B], bonus [B] (-1 for a bad tree), tree_status [B] (may be NULL:
 * BOLE_TREE_BAD_SIZE, BAD_PARENT or BAD_TOKEN; a bad tree accepts nothing). accepted_idx
 * and accepted_len feed bole_commit_path directly.
 */
enum { BOLE_ACCEPT_GREEDY = 0, BOLE_ACCEPT_SAMPLE = 1 };

typedef struct {
    int32_t batch;        /* B >= 0 */
    int32_t total_nodes;  /* T >= 0 */
    int32_t vocab;        /* V >= 1 */
    int32_t max_path;     /* 1..64, row stride of accepted_idx */
    int32_t mode;         /* BOLE_ACCEPT_* */
} bole_accept_dims_t;

BOLE_API bole_status_t bole_tree_accept(const float *p_ctx, const float *p_node,
                               const float *q_ctx, const float *q_node,
                               const int32_t *parent, const int32_t *token,
                               const int32_t *node_offsets, const float *u_node,
                               const float *u_bonus, const bole_accept_dims_t *dims,
                               int32_t *accepted_idx,
                               int32_t *accepted_len, int32_t *bonus, int32_t *tree_status,
                               bole_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* BOLE_H */
