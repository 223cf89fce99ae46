// launch.h - internal host launchers behind the C ABI (not exported).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bole.h"

namespace bole {

constexpr int kMaxTreeNodesHost = 64;  // nodes per tree: one wavefront, one 64-bit mask

// Layers of one launch (blockIdx.y = layer), passed by value as a kernel argument: the
// kernels read their layer's pointers from the argument segment, no table in memory.
constexpr int kLayersPerLaunch = 16;
struct LayerTable {
    bole_layer_t l[kLayersPerLaunch];
};

// The previous step's tree and accepted path, shared by the layers of a lazy commit.
struct PrevPath {
    const int32_t *parent, *node_offsets, *accepted_idx, *accepted_len;
    int32_t *path_nodes, *tree_status;
};

hipError_t launch_prepare(const int32_t *parent, const int32_t *node_offsets, const float *gate,
                          const bole_dims_t &d, int32_t *depth, uint64_t *mask, float *cumlog,
                          int32_t *tree_status, hipStream_t stream);

hipError_t launch_verify_generic(const float *H0, const void *q, const void *k, const void *v,
                                 const float *gate, const int32_t *parent,
                                 const int32_t *node_offsets, float *out, const bole_dims_t &d,
                                 int32_t *tree_status, hipStream_t stream);

// Launchers below take nl <= kLayersPerLaunch layers sharing their trees; statuses and
// path rows are written once.

// True when the matrix-core verify kernel covers this request (every layer).
bool verify_mfma_applies(const bole_dims_t &d, const bole_layer_t *layers, int nl);

hipError_t launch_verify_mfma(const bole_layer_t *layers, int nl, const int32_t *parent,
                              const int32_t *node_offsets, const bole_dims_t &d,
                              int32_t *tree_status, hipStream_t stream);

// True when the matrix-core vector-gate verify kernel covers this request.
bool verify_vec_applies(const bole_dims_t &d, const void *H0, const void *q, const void *k,
                        const void *v, const void *gate, const void *out);

hipError_t launch_verify_vec(const bole_layer_t *layers, int nl, const int32_t *parent,
                             const int32_t *node_offsets, const bole_dims_t &d,
                             int32_t *tree_status, hipStream_t stream);

// The vector-gate kernel with the previous step's commit folded in; applies to a layer
// when its verify does and the previous step's factors have the same shapes and 16-byte
// rows.
bool verify_vec_lazy_applies(const bole_dims_t &d, const bole_dims_t &pd, const bole_layer_t &y);

hipError_t launch_verify_vec_lazy(const bole_layer_t *layers, int nl, const PrevPath &prev,
                                  const bole_dims_t &pd, const int32_t *parent,
                                  const int32_t *node_offsets, const bole_dims_t &d,
                                  int32_t *tree_status, hipStream_t stream);

// True when the one-pass lazy commit + verify kernel covers this pair of steps.
bool verify_lazy_applies(const bole_dims_t &d, const bole_dims_t &pd, const bole_layer_t *layers,
                         int nl);

hipError_t launch_verify_lazy_commit(const bole_layer_t *layers, int nl, const PrevPath &prev,
                                     const bole_dims_t &pd, const int32_t *parent,
                                     const int32_t *node_offsets, const bole_dims_t &d,
                                     int32_t *tree_status, hipStream_t stream);

hipError_t launch_verify_naive(const float *H0, const void *q, const void *k, const void *v,
                               const float *gate, const int32_t *parent,
                               const int32_t *node_offsets, float *out, float *states,
                               const bole_dims_t &d, int32_t *tree_status, hipStream_t stream);

// Commit of each layer's k, v, gate along the shared accepted paths. gate_check (may be
// NULL): per-tree gate statuses written by a kGateReset pass; a tree marked
// BOLE_TREE_BAD_GATE there (and otherwise valid) keeps its state and gets that status.
hipError_t launch_commit(const bole_layer_t *layers, int nl, const int32_t *parent,
                         const int32_t *node_offsets, const int32_t *accepted_idx,
                         const int32_t *accepted_len, const bole_dims_t &d, int32_t *path_nodes,
                         int32_t *tree_status, const int32_t *gate_check, hipStream_t stream);

// Gate-domain check (validate.hip), for BOLE_FLAG_VALIDATE_GATES. Modes: kGateDetect marks
// structurally valid trees with a non-finite or <= 0 gate BOLE_TREE_BAD_GATE; with
// kGateReset it also writes BOLE_TREE_OK for every other tree; kGateFill writes NaN over
// every layer's output rows of the trees marked BOLE_TREE_BAD_GATE.
enum { kGateDetect = 1, kGateReset = 2, kGateFill = 4 };
hipError_t launch_gate_check(const bole_layer_t *layers, int num_layers, const int32_t *parent,
                             const int32_t *node_offsets, const bole_dims_t &d,
                             int32_t *tree_status, int mode, hipStream_t stream);

// Draft-tree construction (tree_build.hip).
bool build_dims_ok(const bole_build_dims_t &d);
size_t build_workspace_bytes(const bole_build_dims_t &d);
// The library-held workspace of bole_build_tree_noalloc on the current GPU (its device
// address, looked up on the first call on that GPU).
constexpr size_t kBuildScratchBytes = (size_t)4 << 20;
hipError_t build_scratch(void **out);
hipError_t launch_build_tree(const float *marginals, const float *cost, float l_ar,
                             void *workspace, const bole_build_dims_t &d, int32_t *node_offsets,
                             int32_t *parent, int32_t *token, float *rho, float *speedup,
                             hipStream_t stream);

// Tree acceptance (tree_accept.hip).
hipError_t launch_tree_accept(const float *p_ctx, const float *p_node, const float *q_ctx,
                              const float *q_node, const int32_t *parent, const int32_t *token,
                              const int32_t *node_offsets, const float *u_node,
                              const float *u_bonus, const bole_accept_dims_t &d,
                              int32_t *accepted_idx,
                              int32_t *accepted_len, int32_t *bonus, int32_t *tree_status,
                              hipStream_t stream);

}  // namespace bole
