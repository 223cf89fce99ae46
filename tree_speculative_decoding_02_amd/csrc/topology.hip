// topology.hip - the tree-topology preprocessor exported as bole_tree_prepare.
//
// One 64-lane workgroup per tree; lane i is tree-local node i. It writes depth,
// the ancestor-or-self mask and the cumulative log-decay. Depth and mask come from
// the same pointer-doubling device code that the verify and commit kernels run
// inline, so this export shows bit for bit the topology those kernels use. The scalar
// cumulative log-decay is the same doubling sum that the generic verify kernel uses
// (the matrix-core kernel keeps the same sum in base 2).
#include "bole_device.h"
#include "launch.h"

namespace bole {

template <bool VEC>
__global__ __launch_bounds__(64) void prepare_kernel(
    const int32_t *__restrict__ parent, const int32_t *__restrict__ node_offsets,
    const float *__restrict__ gate, int32_t *__restrict__ depth, uint64_t *__restrict__ mask,
    float *__restrict__ cumlog, int32_t *__restrict__ tree_status, int H, int DK, int T,
    int max_n) {
    const int b = blockIdx.x;
    const int lane = lane_id();
    const TreeRange tr = tree_range(node_offsets, b, T, max_n);
    if (tr.status != BOLE_TREE_OK) {
        if (lane == 0 && tree_status) tree_status[b] = tr.status;
        return;
    }
    const int lo = tr.lo, n = tr.n;
    const int p_raw = lane < n ? parent[lo + lane] : -1;
    const WaveTopo t = wave_topology_p(p_raw, n);
    if (lane == 0 && tree_status) tree_status[b] = t.bad;
    if (lane < n) {
        if (depth) depth[lo + lane] = t.depth;
        if (mask) mask[lo + lane] = t.mask;
    }
    if (!cumlog) return;
    for (int h = 0; h < H; ++h) {
        if (!VEC) {
            const float lg = (lane < n && !t.bad) ? logf(gate[(size_t)(lo + lane) * H + h]) : 0.f;
            const float L = wave_topology_cumlog(p_raw, lg, n).L;
            if (lane < n) cumlog[(size_t)(lo + lane) * H + h] = L;
        } else {
            for (int c = 0; c < DK; ++c) {
                // node j's log-gate for channel c, read by every lane (same address)
                float L = 0.f;
                for (int j = 0; j < n; ++j) {
                    const float x = t.bad ? 0.f : logf(gate[((size_t)(lo + j) * H + h) * DK + c]);
                    if ((t.mask >> j) & 1ull) L += x;
                }
                if (lane < n) cumlog[((size_t)(lo + lane) * H + h) * DK + c] = L;
            }
        }
    }
}

hipError_t launch_prepare(const int32_t *parent, const int32_t *node_offsets, const float *gate,
                          const bole_dims_t &d, int32_t *depth, uint64_t *mask, float *cumlog,
                          int32_t *tree_status, hipStream_t stream) {
    const dim3 grid(d.batch), block(64);
    if (d.gate_kind == BOLE_GATE_VECTOR)
        prepare_kernel<true><<<grid, block, 0, stream>>>(parent, node_offsets, gate, depth, mask,
                                                         cumlog, tree_status, d.heads, d.d_k,
                                                         d.total_nodes, max_tree_nodes(d.flags));
    else
        prepare_kernel<false><<<grid, block, 0, stream>>>(parent, node_offsets, gate, depth, mask,
                                                          cumlog, tree_status, d.heads, d.d_k,
                                                          d.total_nodes, max_tree_nodes(d.flags));
    return hipGetLastError();
}

}  // namespace bole
