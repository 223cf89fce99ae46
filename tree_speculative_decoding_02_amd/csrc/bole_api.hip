// bole_api.hip - the exported C ABI (declared in include/bole.h): host-side argument
// checks and kernel selection. No allocation, no synchronisation: every entry point
// validates what the host can see, then launches onto the caller's stream.
#include <hip/hip_runtime.h>

#include "bole.h"
#include "launch.h"

namespace {

enum { kOpVerify = 0, kOpCommit = 1, kOpPrepare = 2 };

bole_status_t from_hip(hipError_t e) { return e == hipSuccess ? BOLE_OK : BOLE_ERR_HIP; }

// Verify kernel choice for checked arguments: matrix cores when they cover the request.
hipError_t dispatch_verify(const float *H0, const void *q, const void *k, const void *v,
                           const float *gate, const int32_t *parent, const int32_t *node_offsets,
                           float *out, const bole_dims_t &d, int32_t *tree_status,
                           hipStream_t s) {
    if (bole::verify_mfma_applies(d, H0, q, k, v, out))
        return bole::launch_verify_mfma(H0, q, k, v, gate, parent, node_offsets, out, d,
                                        tree_status, s);
    if (bole::verify_vec_applies(d, H0, q, k, v, gate, out))
        return bole::launch_verify_vec(H0, q, k, v, gate, parent, node_offsets, out, d,
                                       tree_status, s);
    return bole::launch_verify_generic(H0, q, k, v, gate, parent, node_offsets, out, d,
                                       tree_status, s);
}

}  // namespace

extern "C" {

int32_t bole_max_tree_nodes(void) { return bole::kMaxTreeNodesHost; }

const char *bole_status_string(bole_status_t status) {
    switch (status) {
        case BOLE_OK: return "BOLE_OK";
        case BOLE_ERR_INVALID_VALUE: return "BOLE_ERR_INVALID_VALUE";
        case BOLE_ERR_UNSUPPORTED: return "BOLE_ERR_UNSUPPORTED";
        case BOLE_ERR_HIP: return "BOLE_ERR_HIP";
    }
    return "BOLE_ERR_UNKNOWN";
}

bole_status_t bole_check_dims(const bole_dims_t *d, int32_t op) {
    if (d == nullptr || op < kOpVerify || op > kOpPrepare) return BOLE_ERR_INVALID_VALUE;
    if (d->batch < 0 || d->heads < 1 || d->d_k < 1 || d->d_v < 1 || d->total_nodes < 0)
        return BOLE_ERR_INVALID_VALUE;
    if (d->factor_dtype != BOLE_DTYPE_BF16 && d->factor_dtype != BOLE_DTYPE_F32)
        return BOLE_ERR_INVALID_VALUE;
    if (d->gate_kind != BOLE_GATE_SCALAR && d->gate_kind != BOLE_GATE_VECTOR)
        return BOLE_ERR_INVALID_VALUE;
    if (d->flags & ~(BOLE_FLAG_FORCE_GENERIC | BOLE_FLAG_TREES_LE_32)) return BOLE_ERR_INVALID_VALUE;
    if (op == kOpCommit && d->max_path < 0) return BOLE_ERR_INVALID_VALUE;
    if (d->d_k > 256 || d->d_v > 256) return BOLE_ERR_UNSUPPORTED;
    if (op == kOpVerify && d->gate_kind == BOLE_GATE_VECTOR && d->d_k > 128)
        return BOLE_ERR_UNSUPPORTED;
    if (op == kOpCommit && d->max_path > bole::kMaxTreeNodesHost) return BOLE_ERR_UNSUPPORTED;
    // every packed offset must fit the kernels' 32-bit node indices and 64-bit element offsets
    if ((int64_t)d->batch * d->heads > 0x7fffffffLL) return BOLE_ERR_UNSUPPORTED;
    return BOLE_OK;
}

bole_status_t bole_tree_verify(const float *H0, const void *q, const void *k, const void *v,
                               const float *gate, const int32_t *parent,
                               const int32_t *node_offsets, float *out,
                               const bole_dims_t *dims, int32_t *tree_status,
                               bole_stream_t stream) {
    const bole_status_t st = bole_check_dims(dims, kOpVerify);
    if (st != BOLE_OK) return st;
    const bole_dims_t &d = *dims;
    if (d.batch == 0) return BOLE_OK;
    if (H0 == nullptr || node_offsets == nullptr) return BOLE_ERR_INVALID_VALUE;
    if (d.total_nodes > 0 && (q == nullptr || k == nullptr || v == nullptr || gate == nullptr ||
                              parent == nullptr || out == nullptr))
        return BOLE_ERR_INVALID_VALUE;
    return from_hip(dispatch_verify(H0, q, k, v, gate, parent, node_offsets, out, d, tree_status,
                                    reinterpret_cast<hipStream_t>(stream)));
}

bole_status_t bole_tree_verify_lazy_commit(
    float *H0, const bole_factors_t *prev, const int32_t *prev_accepted_idx,
    const int32_t *prev_accepted_len, const bole_dims_t *prev_dims, int32_t *prev_path_nodes,
    int32_t *prev_tree_status, const void *q, const void *k, const void *v, const float *gate,
    const int32_t *parent, const int32_t *node_offsets, float *out, const bole_dims_t *dims,
    int32_t *tree_status, bole_stream_t stream) {
    bole_status_t st = bole_check_dims(dims, kOpVerify);
    if (st != BOLE_OK) return st;
    st = bole_check_dims(prev_dims, kOpCommit);
    if (st != BOLE_OK) return st;
    const bole_dims_t &d = *dims, &pd = *prev_dims;
    // both steps describe the same layer: only the trees and the path may differ
    if (pd.batch != d.batch || pd.heads != d.heads || pd.d_k != d.d_k || pd.d_v != d.d_v ||
        pd.factor_dtype != d.factor_dtype || pd.gate_kind != d.gate_kind)
        return BOLE_ERR_INVALID_VALUE;
    if (d.batch == 0) return BOLE_OK;
    if (H0 == nullptr || node_offsets == nullptr || prev == nullptr ||
        prev->node_offsets == nullptr || prev_accepted_len == nullptr)
        return BOLE_ERR_INVALID_VALUE;
    if (d.total_nodes > 0 && (q == nullptr || k == nullptr || v == nullptr || gate == nullptr ||
                              parent == nullptr || out == nullptr))
        return BOLE_ERR_INVALID_VALUE;
    if (pd.max_path > 0 && prev_accepted_idx == nullptr) return BOLE_ERR_INVALID_VALUE;
    if (pd.total_nodes > 0 && (prev->k == nullptr || prev->v == nullptr ||
                               prev->gate == nullptr || prev->parent == nullptr))
        return BOLE_ERR_INVALID_VALUE;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (bole::verify_lazy_applies(d, pd, H0, q, k, v, out, *prev))
        return from_hip(bole::launch_verify_lazy_commit(
            H0, *prev, prev_accepted_idx, prev_accepted_len, pd, prev_path_nodes,
            prev_tree_status, q, k, v, gate, parent, node_offsets, out, d, tree_status, s));
    // every other shape: the two steps as separate launches, in stream order
    const hipError_t e = bole::launch_commit(H0, *prev, prev_accepted_idx, prev_accepted_len, pd,
                                             prev_path_nodes, prev_tree_status, s);
    if (e != hipSuccess) return from_hip(e);
    return from_hip(dispatch_verify(H0, q, k, v, gate, parent, node_offsets, out, d, tree_status, s));
}

bole_status_t bole_tree_verify_naive(const float *H0, const void *q, const void *k,
                                     const void *v, const float *gate, const int32_t *parent,
                                     const int32_t *node_offsets, float *out, float *states,
                                     const bole_dims_t *dims, int32_t *tree_status,
                                     bole_stream_t stream) {
    const bole_status_t st = bole_check_dims(dims, kOpVerify);
    if (st != BOLE_OK) return st;
    const bole_dims_t &d = *dims;
    if (d.batch == 0) return BOLE_OK;
    if (H0 == nullptr || node_offsets == nullptr) return BOLE_ERR_INVALID_VALUE;
    if (d.total_nodes > 0 && (q == nullptr || k == nullptr || v == nullptr || gate == nullptr ||
                              parent == nullptr || out == nullptr || states == nullptr))
        return BOLE_ERR_INVALID_VALUE;
    return from_hip(bole::launch_verify_naive(H0, q, k, v, gate, parent, node_offsets, out, states,
                                              d, tree_status, reinterpret_cast<hipStream_t>(stream)));
}

bole_status_t bole_commit_path(float *H0, const bole_factors_t *factors,
                               const int32_t *accepted_idx, const int32_t *accepted_len,
                               const bole_dims_t *dims, int32_t *path_nodes,
                               int32_t *tree_status, bole_stream_t stream) {
    const bole_status_t st = bole_check_dims(dims, kOpCommit);
    if (st != BOLE_OK) return st;
    const bole_dims_t &d = *dims;
    if (d.batch == 0) return BOLE_OK;
    if (H0 == nullptr || factors == nullptr || factors->node_offsets == nullptr ||
        accepted_len == nullptr)
        return BOLE_ERR_INVALID_VALUE;
    if (d.max_path > 0 && accepted_idx == nullptr) return BOLE_ERR_INVALID_VALUE;
    if (d.total_nodes > 0 && (factors->k == nullptr || factors->v == nullptr ||
                              factors->gate == nullptr || factors->parent == nullptr))
        return BOLE_ERR_INVALID_VALUE;
    return from_hip(bole::launch_commit(H0, *factors, accepted_idx, accepted_len, d, path_nodes,
                                        tree_status, reinterpret_cast<hipStream_t>(stream)));
}

bole_status_t bole_tree_prepare(const int32_t *parent, const int32_t *node_offsets,
                                const float *gate, const bole_dims_t *dims, int32_t *depth,
                                uint64_t *mask, float *cumlog, int32_t *tree_status,
                                bole_stream_t stream) {
    const bole_status_t st = bole_check_dims(dims, kOpPrepare);
    if (st != BOLE_OK) return st;
    const bole_dims_t &d = *dims;
    if (d.batch == 0) return BOLE_OK;
    if (node_offsets == nullptr) return BOLE_ERR_INVALID_VALUE;
    if (d.total_nodes > 0 && parent == nullptr) return BOLE_ERR_INVALID_VALUE;
    if (cumlog != nullptr && d.total_nodes > 0 && gate == nullptr) return BOLE_ERR_INVALID_VALUE;
    return from_hip(bole::launch_prepare(parent, node_offsets, gate, d, depth, mask, cumlog,
                                         tree_status, reinterpret_cast<hipStream_t>(stream)));
}

}  // extern "C"
