// validate.hip - the gate-domain check behind BOLE_FLAG_VALIDATE_GATES.
//
// The closed form of the Bole summary page, section 1, takes logarithms of the gates
// (each S_i = a_i I or diag(g_i) is a decay, finite and > 0). A gate outside that domain
// cannot move any index or memory access (tree structure and paths decide those), but it
// voids the results of its tree. Under the flag:
//  - verify: after the verify kernels, DETECT marks every structurally valid tree with a
//    bad gate (any layer, head or channel) BOLE_TREE_BAD_GATE in tree_status, then FILL
//    writes NaN over that tree's output rows in every layer;
//  - commit: before the commit kernels, DETECT_RESET writes every tree's gate status
//    (OK or BAD_GATE), and the commit kernels keep the state of a BAD_GATE sequence in
//    every layer.
// One 256-thread workgroup per tree; wavefront 0 re-checks the tree's offsets and parent
// links with the rules the verify and commit kernels use, so that a tree they already
// reported bad (size, parent) keeps that status.
#include "bole_device.h"
#include "launch.h"

namespace bole {

constexpr int kCheckThreads = 256;

__global__ __launch_bounds__(kCheckThreads) void gate_check_kernel(
    const LayerTable lt, int nl, const int32_t *__restrict__ parent,
    const int32_t *__restrict__ node_offsets, int32_t *__restrict__ tree_status, int H,
    int GW, int DV, int T, int max_n, int mode) {
    __shared__ int s_ok, s_lo, s_n;
    const int b = blockIdx.x, tid = threadIdx.x;
    if (tid < 64) {
        const TreeRange tr = tree_range(node_offsets, b, T, max_n);
        bool ok = tr.status == BOLE_TREE_OK;
        const int n = ok ? tr.n : 0;
        const int p = tid < n ? parent[tr.lo + tid] : -1;
        if (__any(tid < n && (p < -1 || p >= tid))) ok = false;
        if (tid == 0) {
            s_ok = ok;
            s_lo = tr.lo;
            s_n = n;
        }
    }
    __syncthreads();
    const bool ok = s_ok;
    const size_t lo = (size_t)s_lo, n = (size_t)s_n;
    if (mode & kGateFill) {
        // NaN over every layer's rows of a tree marked BAD_GATE (by the DETECT passes)
        if (tree_status[b] != BOLE_TREE_BAD_GATE) return;
        const size_t cnt = n * (size_t)H * (size_t)DV;
        for (int l = 0; l < nl; ++l) {
            float *o = lt.l[l].out + lo * (size_t)H * (size_t)DV;
            for (size_t e = tid; e < cnt; e += kCheckThreads) o[e] = __builtin_nanf("");
        }
        return;
    }
    bool bad = false;
    if (ok) {
        const size_t cnt = n * (size_t)H * (size_t)GW;
        for (int l = 0; l < nl; ++l) {
            const float *g = lt.l[l].gate + lo * (size_t)H * (size_t)GW;
            for (size_t e = tid; e < cnt; e += kCheckThreads) {
                const float x = g[e];
                bad |= !(x > 0.f && x <= 3.402823466e38f);  // NaN fails both tests
            }
        }
    }
    bad = __syncthreads_or(bad);
    if (tid == 0) {
        if (bad) tree_status[b] = BOLE_TREE_BAD_GATE;
        else if (mode & kGateReset) tree_status[b] = BOLE_TREE_OK;
    }
}

hipError_t launch_gate_check(const bole_layer_t *layers, int num_layers, const int32_t *parent,
                             const int32_t *node_offsets, const bole_dims_t &d,
                             int32_t *tree_status, int mode, hipStream_t stream) {
    const int GW = d.gate_kind == BOLE_GATE_VECTOR ? d.d_k : 1;
    for (int l0 = 0; l0 < num_layers; l0 += kLayersPerLaunch) {
        const int nl = num_layers - l0 < kLayersPerLaunch ? num_layers - l0 : kLayersPerLaunch;
        LayerTable lt = {};
        for (int l = 0; l < nl; ++l) lt.l[l] = layers[l0 + l];
        // only the first chunk resets: later chunks may only add BAD_GATE
        const int m = l0 == 0 ? mode : (mode & ~kGateReset);
        gate_check_kernel<<<dim3((unsigned)d.batch), dim3(kCheckThreads), 0, stream>>>(
            lt, nl, parent, node_offsets, tree_status, d.heads, GW, d.d_v, d.total_nodes,
            max_tree_nodes(d.flags), m);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace bole
