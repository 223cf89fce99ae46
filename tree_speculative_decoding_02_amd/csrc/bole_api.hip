// bole_api.hip - the exported C ABI (declared in include/bole.h): host-side argument
// checks and kernel selection. No allocation, no synchronisation: every entry point
// validates what the host can see, then launches onto the caller's stream.
#include <hip/hip_runtime.h>

#include "bole.h"
#include "launch.h"

namespace {

enum { kOpVerify = 0, kOpCommit = 1, kOpPrepare = 2 };

bole_status_t from_hip(hipError_t e) { return e == hipSuccess ? BOLE_OK : BOLE_ERR_HIP; }

using bole::kLayersPerLaunch;

// Layers l0 .. l0 + nl - 1 into `out` (nl <= kLayersPerLaunch); with `prev`, each layer's
// k, v, gate replaced by the previous step's (the commit half of a lazy step).
int chunk(const bole_layer_t *layers, int num_layers, int l0, bool prev, bole_layer_t *out) {
    const int nl = num_layers - l0 < kLayersPerLaunch ? num_layers - l0 : kLayersPerLaunch;
    for (int l = 0; l < nl; ++l) {
        out[l] = layers[l0 + l];
        if (prev) {
            out[l].k = out[l].prev_k;
            out[l].v = out[l].prev_v;
            out[l].gate = out[l].prev_gate;
        }
    }
    return nl;
}

// Gate-domain passes (BOLE_FLAG_VALIDATE_GATES) over every layer, kLayersPerLaunch at a
// time; kGateReset applies to the first chunk only, so later chunks can only add
// BOLE_TREE_BAD_GATE.
hipError_t gate_pass(const bole_layer_t *layers, int num_layers, bool prev, const int32_t *parent,
                     const int32_t *node_offsets, const bole_dims_t &d, int32_t *tree_status,
                     int mode, hipStream_t s) {
    bole_layer_t ch[kLayersPerLaunch];
    for (int l0 = 0; l0 < num_layers; l0 += kLayersPerLaunch) {
        const int nl = chunk(layers, num_layers, l0, prev, ch);
        const hipError_t e = bole::launch_gate_check(ch, nl, parent, node_offsets, d, tree_status,
                                                     l0 == 0 ? mode : (mode & ~bole::kGateReset), s);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

// Verify of checked layers, kLayersPerLaunch at a time: the scalar-gate or vector-gate
// matrix-core kernel when it covers every layer of the chunk (one launch), else the
// vector-gate or plain kernel layer by layer. Per-tree outputs come from the first launch
// only. Under BOLE_FLAG_VALIDATE_GATES the gate check
// follows: every layer's gates, then NaN rows of the trees found bad, in every layer.
hipError_t dispatch_verify(const bole_layer_t *layers, int num_layers, const int32_t *parent,
                           const int32_t *node_offsets, const bole_dims_t &d,
                           int32_t *tree_status, hipStream_t s) {
    for (int l0 = 0; l0 < num_layers; l0 += kLayersPerLaunch) {
        const bole_layer_t *ch = layers + l0;
        const int nl = num_layers - l0 < kLayersPerLaunch ? num_layers - l0 : kLayersPerLaunch;
        int32_t *ts = l0 == 0 ? tree_status : nullptr;
        hipError_t e = hipSuccess;
        bool vec = true;
        for (int l = 0; l < nl; ++l) {
            const bole_layer_t &y = ch[l];
            vec = vec && bole::verify_vec_applies(d, y.H0, y.q, y.k, y.v, y.gate, y.out);
        }
        if (bole::verify_mfma_applies(d, ch, nl)) {
            e = bole::launch_verify_mfma(ch, nl, parent, node_offsets, d, ts, s);
        } else if (vec) {
            e = bole::launch_verify_vec(ch, nl, parent, node_offsets, d, ts, s);
        } else {
            for (int l = 0; l < nl && e == hipSuccess; ++l) {
                const bole_layer_t &y = ch[l];
                int32_t *tl = l == 0 ? ts : nullptr;
                e = bole::verify_vec_applies(d, y.H0, y.q, y.k, y.v, y.gate, y.out)
                        ? bole::launch_verify_vec(&y, 1, parent, node_offsets, d, tl, s)
                        : bole::launch_verify_generic(y.H0, y.q, y.k, y.v, y.gate, parent,
                                                      node_offsets, y.out, d, tl, s);
            }
        }
        if (e != hipSuccess) return e;
    }
    if (d.flags & BOLE_FLAG_VALIDATE_GATES) {
        hipError_t e = gate_pass(layers, num_layers, false, parent, node_offsets, d, tree_status,
                                 bole::kGateDetect, s);
        if (e == hipSuccess)
            e = gate_pass(layers, num_layers, false, parent, node_offsets, d, tree_status,
                          bole::kGateFill, s);
        return e;
    }
    return hipSuccess;
}

// Commit of checked layers (with `prev`: of the previous step's factors), kLayersPerLaunch
// at a time. Under BOLE_FLAG_VALIDATE_GATES every tree's gate status over all layers is
// written first, and the commit kernels keep the state of the trees marked bad.
hipError_t dispatch_commit(const bole_layer_t *layers, int num_layers, bool prev,
                           const int32_t *parent, const int32_t *node_offsets,
                           const int32_t *accepted_idx, const int32_t *accepted_len,
                           const bole_dims_t &d, int32_t *path_nodes, int32_t *tree_status,
                           hipStream_t s) {
    const int32_t *gate_check = nullptr;
    if (d.flags & BOLE_FLAG_VALIDATE_GATES) {
        const hipError_t e = gate_pass(layers, num_layers, prev, parent, node_offsets, d,
                                       tree_status, bole::kGateDetect | bole::kGateReset, s);
        if (e != hipSuccess) return e;
        gate_check = tree_status;
    }
    bole_layer_t ch[kLayersPerLaunch];
    for (int l0 = 0; l0 < num_layers; l0 += kLayersPerLaunch) {
        const int nl = chunk(layers, num_layers, l0, prev, ch);
        const hipError_t e = bole::launch_commit(ch, nl, parent, node_offsets, accepted_idx,
                                                 accepted_len, d, l0 == 0 ? path_nodes : nullptr,
                                                 l0 == 0 ? tree_status : nullptr, gate_check, s);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

// One pass per chunk where the lazy kernel covers it; elsewhere the previous step's
// commit (on prev_k, prev_v, prev_gate) then this step's verify, chunk by chunk. Under
// BOLE_FLAG_VALIDATE_GATES (either step) the two run as separate calls over the whole
// stack, each with its gate check.
hipError_t dispatch_lazy(const bole_layer_t *layers, int num_layers, const bole::PrevPath &prev,
                         const bole_dims_t &pd, const int32_t *parent, const int32_t *node_offsets,
                         const bole_dims_t &d, int32_t *tree_status, hipStream_t s) {
    if ((d.flags | pd.flags) & BOLE_FLAG_VALIDATE_GATES) {
        hipError_t e = dispatch_commit(layers, num_layers, true, prev.parent, prev.node_offsets,
                                       prev.accepted_idx, prev.accepted_len, pd, prev.path_nodes,
                                       prev.tree_status, s);
        if (e == hipSuccess)
            e = dispatch_verify(layers, num_layers, parent, node_offsets, d, tree_status, s);
        return e;
    }
    bole_layer_t pl[kLayersPerLaunch];
    for (int l0 = 0; l0 < num_layers; l0 += kLayersPerLaunch) {
        const bole_layer_t *ch = layers + l0;
        const int nl = chunk(layers, num_layers, l0, true, pl);
        bole::PrevPath pp = prev;
        if (l0 > 0) pp.path_nodes = pp.tree_status = nullptr;
        int32_t *ts = l0 == 0 ? tree_status : nullptr;
        hipError_t e = hipSuccess;
        bool vec = true;  // the vector-gate kernel's one-pass form covers every layer
        for (int l = 0; l < nl; ++l) vec = vec && bole::verify_vec_lazy_applies(d, pd, ch[l]);
        if (bole::verify_lazy_applies(d, pd, ch, nl)) {
            e = bole::launch_verify_lazy_commit(ch, nl, pp, pd, parent, node_offsets, d, ts, s);
        } else if (vec) {
            e = bole::launch_verify_vec_lazy(ch, nl, pp, pd, parent, node_offsets, d, ts, s);
        } else {
            e = bole::launch_commit(pl, nl, pp.parent, pp.node_offsets, pp.accepted_idx,
                                    pp.accepted_len, pd, pp.path_nodes, pp.tree_status, nullptr, s);
            if (e == hipSuccess) e = dispatch_verify(ch, nl, parent, node_offsets, d, ts, s);
        }
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

// BOLE_FLAG_VALIDATE_GATES reports through tree_status, so it needs one.
bool validate_ok(const bole_dims_t &d, const int32_t *tree_status) {
    return !(d.flags & BOLE_FLAG_VALIDATE_GATES) || tree_status != nullptr;
}

// Host-visible checks shared by the entry points. `need_out`: verify outputs; `distinct`:
// which per-layer buffer must differ between layers (0 none, 1 H0, 2 out, 3 both).
bool layers_ok(const bole_layer_t *layers, int num_layers, const bole_dims_t &d, bool verify,
               bool prev, const bole_dims_t *pd, int distinct) {
    if (layers == nullptr || num_layers < 1) return false;
    for (int l = 0; l < num_layers; ++l) {
        const bole_layer_t &y = layers[l];
        if (y.H0 == nullptr) return false;
        if (d.total_nodes > 0 && (y.k == nullptr || y.v == nullptr || y.gate == nullptr))
            return false;
        if (verify && d.total_nodes > 0 && (y.q == nullptr || y.out == nullptr)) return false;
        if (prev && pd->total_nodes > 0 &&
            (y.prev_k == nullptr || y.prev_v == nullptr || y.prev_gate == nullptr))
            return false;
        for (int m = 0; m < l; ++m) {
            if ((distinct & 1) && layers[m].H0 == y.H0) return false;
            if ((distinct & 2) && y.out != nullptr && layers[m].out == y.out) return false;
        }
    }
    return true;
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
        case BOLE_ERR_BAD_TREE: return "BOLE_ERR_BAD_TREE";
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
    if (d->flags & ~(BOLE_FLAG_FORCE_GENERIC | BOLE_FLAG_TREES_LE_32 | BOLE_FLAG_VALIDATE_GATES))
        return BOLE_ERR_INVALID_VALUE;
    if (op == kOpCommit && d->max_path < 0) return BOLE_ERR_INVALID_VALUE;
    if (d->d_k > 256 || d->d_v > 256) return BOLE_ERR_UNSUPPORTED;
    if (op == kOpCommit && d->max_path > bole::kMaxTreeNodesHost) return BOLE_ERR_UNSUPPORTED;
    // every packed offset must fit the kernels' 32-bit node indices and 64-bit element offsets
    if ((int64_t)d->batch * d->heads > 0x7fffffffLL) return BOLE_ERR_UNSUPPORTED;
    return BOLE_OK;
}

size_t bole_workspace_bytes(const bole_dims_t *dims) {
    (void)dims;
    return 0;
}

bole_status_t bole_read_status(const int32_t *tree_status, int32_t batch, int32_t *host_status,
                               bole_stream_t stream) {
    if (batch < 0 || (batch > 0 && tree_status == nullptr)) return BOLE_ERR_INVALID_VALUE;
    const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    // into the caller's array, or through a small buffer on the stack: nothing allocated
    int32_t buf[256];
    bool bad = false;
    for (int32_t b0 = 0; b0 < batch; b0 += 256) {
        const int32_t nb = batch - b0 < 256 ? batch - b0 : 256;
        int32_t *dst = host_status ? host_status + b0 : buf;
        if (hipMemcpyAsync(dst, tree_status + b0, sizeof(int32_t) * (size_t)nb,
                           hipMemcpyDeviceToHost, s) != hipSuccess ||
            hipStreamSynchronize(s) != hipSuccess)
            return BOLE_ERR_HIP;
        for (int32_t i = 0; i < nb; ++i) bad = bad || dst[i] != BOLE_TREE_OK;
    }
    return bad ? BOLE_ERR_BAD_TREE : BOLE_OK;
}

bole_status_t bole_tree_verify_layers(const bole_layer_t *layers, int32_t num_layers,
                                      const int32_t *parent, const int32_t *node_offsets,
                                      const bole_dims_t *dims, int32_t *tree_status,
                                      bole_stream_t stream) {
    const bole_status_t st = bole_check_dims(dims, kOpVerify);
    if (st != BOLE_OK) return st;
    const bole_dims_t &d = *dims;
    if (layers == nullptr || num_layers < 1) return BOLE_ERR_INVALID_VALUE;
    if (d.batch == 0) return BOLE_OK;
    if (node_offsets == nullptr || (d.total_nodes > 0 && parent == nullptr) ||
        !layers_ok(layers, num_layers, d, true, false, nullptr, 2) || !validate_ok(d, tree_status))
        return BOLE_ERR_INVALID_VALUE;
    return from_hip(dispatch_verify(layers, num_layers, parent, node_offsets, d, tree_status,
                                    reinterpret_cast<hipStream_t>(stream)));
}

bole_status_t bole_tree_verify(const float *H0, const void *q, const void *k, const void *v,
                               const float *gate, const int32_t *parent,
                               const int32_t *node_offsets, float *out,
                               const bole_dims_t *dims, int32_t *tree_status,
                               bole_stream_t stream) {
    const bole_layer_t y = {const_cast<float *>(H0), q, k, v, gate, out, nullptr, nullptr, nullptr};
    return bole_tree_verify_layers(&y, 1, parent, node_offsets, dims, tree_status, stream);
}

bole_status_t bole_tree_verify_lazy_commit_layers(
    const bole_layer_t *layers, int32_t num_layers, const int32_t *prev_parent,
    const int32_t *prev_node_offsets, const int32_t *prev_accepted_idx,
    const int32_t *prev_accepted_len, const bole_dims_t *prev_dims, int32_t *prev_path_nodes,
    int32_t *prev_tree_status, const int32_t *parent, const int32_t *node_offsets,
    const bole_dims_t *dims, int32_t *tree_status, bole_stream_t stream) {
    bole_status_t st = bole_check_dims(dims, kOpVerify);
    if (st != BOLE_OK) return st;
    st = bole_check_dims(prev_dims, kOpCommit);
    if (st != BOLE_OK) return st;
    const bole_dims_t &d = *dims, &pd = *prev_dims;
    // both steps describe the same layers: only the trees and the path may differ
    if (pd.batch != d.batch || pd.heads != d.heads || pd.d_k != d.d_k || pd.d_v != d.d_v ||
        pd.factor_dtype != d.factor_dtype || pd.gate_kind != d.gate_kind)
        return BOLE_ERR_INVALID_VALUE;
    if (layers == nullptr || num_layers < 1) return BOLE_ERR_INVALID_VALUE;
    if (d.batch == 0) return BOLE_OK;
    if (node_offsets == nullptr || prev_node_offsets == nullptr || prev_accepted_len == nullptr)
        return BOLE_ERR_INVALID_VALUE;
    if ((d.total_nodes > 0 && parent == nullptr) || (pd.total_nodes > 0 && prev_parent == nullptr))
        return BOLE_ERR_INVALID_VALUE;
    if (pd.max_path > 0 && prev_accepted_idx == nullptr) return BOLE_ERR_INVALID_VALUE;
    if (!layers_ok(layers, num_layers, d, true, true, &pd, 3) || !validate_ok(d, tree_status) ||
        !validate_ok(pd, prev_tree_status))
        return BOLE_ERR_INVALID_VALUE;
    const bole::PrevPath prev = {prev_parent, prev_node_offsets, prev_accepted_idx,
                                 prev_accepted_len, prev_path_nodes, prev_tree_status};
    return from_hip(dispatch_lazy(layers, num_layers, prev, pd, parent, node_offsets, d,
                                  tree_status, reinterpret_cast<hipStream_t>(stream)));
}

bole_status_t bole_tree_verify_lazy_commit(
    float *H0, const bole_factors_t *prev, const int32_t *prev_accepted_idx,
    const int32_t *prev_accepted_len, const bole_dims_t *prev_dims, int32_t *prev_path_nodes,
    int32_t *prev_tree_status, const void *q, const void *k, const void *v, const float *gate,
    const int32_t *parent, const int32_t *node_offsets, float *out, const bole_dims_t *dims,
    int32_t *tree_status, bole_stream_t stream) {
    if (prev == nullptr) {
        // the dims checks still come first, as in every entry point
        bole_status_t st = bole_check_dims(dims, kOpVerify);
        if (st == BOLE_OK) st = bole_check_dims(prev_dims, kOpCommit);
        return st != BOLE_OK ? st : (dims->batch == 0 ? BOLE_OK : BOLE_ERR_INVALID_VALUE);
    }
    const bole_layer_t y = {H0, q, k, v, gate, out, prev->k, prev->v, prev->gate};
    return bole_tree_verify_lazy_commit_layers(&y, 1, prev->parent, prev->node_offsets,
                                               prev_accepted_idx, prev_accepted_len, prev_dims,
                                               prev_path_nodes, prev_tree_status, parent,
                                               node_offsets, dims, tree_status, stream);
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
    if (!validate_ok(d, tree_status)) return BOLE_ERR_INVALID_VALUE;
    const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    hipError_t e = bole::launch_verify_naive(H0, q, k, v, gate, parent, node_offsets, out, states,
                                             d, tree_status, s);
    if (e == hipSuccess && (d.flags & BOLE_FLAG_VALIDATE_GATES)) {
        const bole_layer_t y = {const_cast<float *>(H0), q, k, v, gate, out, nullptr, nullptr, nullptr};
        e = gate_pass(&y, 1, false, parent, node_offsets, d, tree_status, bole::kGateDetect, s);
        if (e == hipSuccess)
            e = gate_pass(&y, 1, false, parent, node_offsets, d, tree_status, bole::kGateFill, s);
    }
    return from_hip(e);
}

bole_status_t bole_commit_path_layers(const bole_layer_t *layers, int32_t num_layers,
                                      const int32_t *parent, const int32_t *node_offsets,
                                      const int32_t *accepted_idx, const int32_t *accepted_len,
                                      const bole_dims_t *dims, int32_t *path_nodes,
                                      int32_t *tree_status, bole_stream_t stream) {
    const bole_status_t st = bole_check_dims(dims, kOpCommit);
    if (st != BOLE_OK) return st;
    const bole_dims_t &d = *dims;
    if (layers == nullptr || num_layers < 1) return BOLE_ERR_INVALID_VALUE;
    if (d.batch == 0) return BOLE_OK;
    if (node_offsets == nullptr || accepted_len == nullptr) return BOLE_ERR_INVALID_VALUE;
    if (d.max_path > 0 && accepted_idx == nullptr) return BOLE_ERR_INVALID_VALUE;
    if ((d.total_nodes > 0 && parent == nullptr) ||
        !layers_ok(layers, num_layers, d, false, false, nullptr, 1) || !validate_ok(d, tree_status))
        return BOLE_ERR_INVALID_VALUE;
    return from_hip(dispatch_commit(layers, num_layers, false, parent, node_offsets, accepted_idx,
                                    accepted_len, d, path_nodes, tree_status,
                                    reinterpret_cast<hipStream_t>(stream)));
}

bole_status_t bole_commit_path(float *H0, const bole_factors_t *factors,
                               const int32_t *accepted_idx, const int32_t *accepted_len,
                               const bole_dims_t *dims, int32_t *path_nodes,
                               int32_t *tree_status, bole_stream_t stream) {
    if (factors == nullptr) {
        const bole_status_t st = bole_check_dims(dims, kOpCommit);
        return st != BOLE_OK ? st : (dims->batch == 0 ? BOLE_OK : BOLE_ERR_INVALID_VALUE);
    }
    const bole_layer_t y = {H0, nullptr, factors->k, factors->v, factors->gate, nullptr,
                            nullptr, nullptr, nullptr};
    return bole_commit_path_layers(&y, 1, factors->parent, factors->node_offsets, accepted_idx,
                                   accepted_len, dims, path_nodes, tree_status, stream);
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
    const bool validate = (d.flags & BOLE_FLAG_VALIDATE_GATES) != 0;
    if (validate && (tree_status == nullptr || (d.total_nodes > 0 && gate == nullptr)))
        return BOLE_ERR_INVALID_VALUE;
    const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    hipError_t e = bole::launch_prepare(parent, node_offsets, gate, d, depth, mask, cumlog,
                                        tree_status, s);
    if (e == hipSuccess && validate) {
        const bole_layer_t y = {nullptr, nullptr, nullptr, nullptr, gate, nullptr, nullptr, nullptr, nullptr};
        e = gate_pass(&y, 1, false, parent, node_offsets, d, tree_status, bole::kGateDetect, s);
    }
    return from_hip(e);
}

size_t bole_build_tree_workspace_size(const bole_build_dims_t *dims) {
    if (dims == nullptr || !bole::build_dims_ok(*dims)) return 0;
    return bole::build_workspace_bytes(*dims);
}

// Checks shared by the two builder entry points (everything but the workspace).
static bole_status_t build_args_ok(const float *marginals, const float *cost, float l_ar,
                            const bole_build_dims_t *dims, const int32_t *node_offsets,
                            const int32_t *parent, const int32_t *token, const float *speedup) {
    if (dims == nullptr) return BOLE_ERR_INVALID_VALUE;
    const bole_build_dims_t &d = *dims;
    if (d.batch < 0 || d.vocab < 1 || d.n_max < 1 || d.depth < 1 ||
        (d.flags & ~BOLE_BUILD_FIXED_BUDGET))
        return BOLE_ERR_INVALID_VALUE;
    if (!bole::build_dims_ok(d)) return BOLE_ERR_UNSUPPORTED;
    if (d.batch == 0) return BOLE_OK;
    const bool fixed = (d.flags & BOLE_BUILD_FIXED_BUDGET) != 0;
    if (marginals == nullptr || node_offsets == nullptr || parent == nullptr || token == nullptr)
        return BOLE_ERR_INVALID_VALUE;
    if (cost == nullptr && (!fixed || speedup != nullptr)) return BOLE_ERR_INVALID_VALUE;
    if (!fixed && !(l_ar > 0.f && l_ar < 3.4e38f)) return BOLE_ERR_INVALID_VALUE;
    return BOLE_OK;
}

bole_status_t bole_build_tree_noalloc(const float *marginals, const float *cost, float l_ar,
                                      const bole_build_dims_t *dims, int32_t *node_offsets,
                                      int32_t *parent, int32_t *token, float *rho,
                                      float *speedup, bole_stream_t stream) {
    const bole_status_t st =
        build_args_ok(marginals, cost, l_ar, dims, node_offsets, parent, token, speedup);
    if (st != BOLE_OK || dims->batch == 0) return st;
    static_assert(bole::kBuildScratchBytes == BOLE_BUILD_NOALLOC_MAX_BYTES, "header limit");
    if (bole::build_workspace_bytes(*dims) > bole::kBuildScratchBytes) return BOLE_ERR_UNSUPPORTED;
    void *ws = nullptr;
    if (bole::build_scratch(&ws) != hipSuccess) return BOLE_ERR_HIP;
    return from_hip(bole::launch_build_tree(marginals, cost, l_ar, ws, *dims, node_offsets,
                                            parent, token, rho, speedup,
                                            reinterpret_cast<hipStream_t>(stream)));
}

bole_status_t bole_build_tree(const float *marginals, const float *cost, float l_ar,
                              void *workspace, size_t workspace_bytes,
                              const bole_build_dims_t *dims, int32_t *node_offsets,
                              int32_t *parent, int32_t *token, float *rho, float *speedup,
                              bole_stream_t stream) {
    const bole_status_t st =
        build_args_ok(marginals, cost, l_ar, dims, node_offsets, parent, token, speedup);
    if (st != BOLE_OK || dims->batch == 0) return st;
    const bole_build_dims_t &d = *dims;
    if (workspace == nullptr || reinterpret_cast<uintptr_t>(workspace) % 16 != 0 ||
        workspace_bytes < bole::build_workspace_bytes(d))
        return BOLE_ERR_INVALID_VALUE;
    return from_hip(bole::launch_build_tree(marginals, cost, l_ar, workspace, d, node_offsets,
                                            parent, token, rho, speedup,
                                            reinterpret_cast<hipStream_t>(stream)));
}

static bool accept_dims_ok(const bole_accept_dims_t &d) {
    return d.batch >= 0 && d.total_nodes >= 0 && d.vocab >= 1 && d.max_path >= 1 &&
           d.max_path <= bole::kMaxTreeNodesHost &&
           (d.mode == BOLE_ACCEPT_GREEDY || d.mode == BOLE_ACCEPT_SAMPLE);
}

bole_status_t bole_tree_accept(const float *p_ctx, const float *p_node, const float *q_ctx,
                               const float *q_node, const int32_t *parent, const int32_t *token,
                               const int32_t *node_offsets, const float *u_node,
                               const float *u_bonus, const bole_accept_dims_t *dims,
                               int32_t *accepted_idx,
                               int32_t *accepted_len, int32_t *bonus, int32_t *tree_status,
                               bole_stream_t stream) {
    if (dims == nullptr || !accept_dims_ok(*dims)) return BOLE_ERR_INVALID_VALUE;
    const bole_accept_dims_t &d = *dims;
    if (d.batch == 0) return BOLE_OK;
    if (p_ctx == nullptr || node_offsets == nullptr || accepted_idx == nullptr ||
        accepted_len == nullptr || bonus == nullptr)
        return BOLE_ERR_INVALID_VALUE;
    if (d.total_nodes > 0 && (p_node == nullptr || parent == nullptr || token == nullptr))
        return BOLE_ERR_INVALID_VALUE;
    if (d.mode == BOLE_ACCEPT_SAMPLE) {
        if (q_ctx == nullptr || u_bonus == nullptr ||
            (d.total_nodes > 0 && (q_node == nullptr || u_node == nullptr)))
            return BOLE_ERR_INVALID_VALUE;
    }
    // row offsets (T + B rows of V) fit the kernels' 64-bit element offsets
    if ((uint64_t)(d.total_nodes + (int64_t)d.batch) * (uint64_t)d.vocab >= (1ull << 62))
        return BOLE_ERR_UNSUPPORTED;
    return from_hip(bole::launch_tree_accept(p_ctx, p_node, q_ctx, q_node, parent, token,
                                             node_offsets, u_node, u_bonus, d,
                                             accepted_idx, accepted_len, bonus, tree_status,
                                             reinterpret_cast<hipStream_t>(stream)));
}

}  // extern "C"
