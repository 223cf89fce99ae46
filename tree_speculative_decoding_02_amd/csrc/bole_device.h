// bole_device.h - device helpers shared by the gfx950 kernels: tree bounds, per-tree
// topology on one 64-lane wavefront, root-first cumulative log-decay, MFMA fragment types.
//
// A draft tree has at most 64 nodes. One wavefront holds the whole tree: lane i is
// tree-local node i. That gives one 64-bit ancestor mask per node and lets every
// topology step be a cross-lane shuffle, with no LDS and no barrier.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bole.h"

namespace bole {

constexpr int kMaxTree = 64;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

__device__ __forceinline__ uint64_t shfl_u64(uint64_t x, int src) {
    const int lo = __shfl(static_cast<int>(static_cast<uint32_t>(x)), src, 64);
    const int hi = __shfl(static_cast<int>(static_cast<uint32_t>(x >> 32)), src, 64);
    return (static_cast<uint64_t>(static_cast<uint32_t>(hi)) << 32) | static_cast<uint32_t>(lo);
}

// Value of x in lane src (src must be wave-uniform; a compile-time constant is best).
__device__ __forceinline__ float readlane_f(float x, int src_uniform) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), src_uniform));
}

// Packed rows [lo, lo + n) of tree b, and whether the offsets describe a valid tree.
struct TreeRange {
    int lo;
    int n;
    int status;
};

// max_n: the largest valid tree (kMaxTree, or 32 under BOLE_FLAG_TREES_LE_32).
__device__ __forceinline__ TreeRange tree_range(const int32_t *node_offsets, int b, int T,
                                                int max_n = kMaxTree) {
    const int lo = node_offsets[b];
    const int hi = node_offsets[b + 1];
    TreeRange r;
    r.lo = lo;
    r.n = hi - lo;
    r.status = (lo < 0 || hi < lo || hi > T || hi - lo > max_n) ? BOLE_TREE_BAD_SIZE
                                                                 : BOLE_TREE_OK;
    return r;
}

__host__ __device__ __forceinline__ int max_tree_nodes(int32_t flags) {
    return (flags & BOLE_FLAG_TREES_LE_32) ? 32 : kMaxTree;
}

// Topology of the tree whose tree-local parent array is par[0 .. n-1], computed by
// the calling wavefront (all 64 lanes active, n <= 64, n wave-uniform). Lane i gets
// the ancestor-or-self mask of node i (bit j set iff node j is on the root-to-i path)
// and its depth (number of nodes on that path). `bad` (wave-uniform) is
// BOLE_TREE_BAD_PARENT if any parent[i] lies outside [-1, i); then masks and depths
// are 0.
//
// The mask is built by pointer doubling. After round r, a lane's mask covers its
// 2^r nearest path nodes, and its `anc` pointer has jumped 2^r levels up. Six rounds
// cover any path of 64 nodes.
struct WaveTopo {
    uint64_t mask;
    int depth;
    int bad;
};

// Same, from the parent index already loaded by lane i (any value for lanes >= n).
// Doubling stops as soon as every lane's pointer has passed a root, so a tree of depth
// d costs ceil(log2 d) rounds.
__device__ __forceinline__ WaveTopo wave_topology_p(int p_loaded, int n) {
    const int lane = lane_id();
    const int p = lane < n ? p_loaded : -1;
    const bool bad_lane = lane < n && (p < -1 || p >= lane);
    WaveTopo t;
    t.bad = __any(bad_lane) ? BOLE_TREE_BAD_PARENT : BOLE_TREE_OK;
    uint64_t m = (lane < n && !t.bad) ? (1ull << lane) : 0ull;
    int anc = (lane < n && !t.bad) ? p : -1;
    for (int r = 0; r < 6 && __any(anc >= 0); ++r) {
        const int src = anc < 0 ? lane : anc;
        const uint64_t m_up = shfl_u64(m, src);
        const int anc_up = __shfl(anc, src, 64);
        if (anc >= 0) {
            m |= m_up;
            anc = anc_up;
        }
    }
    t.mask = m;
    t.depth = __popcll(m);
    return t;
}

__device__ __forceinline__ WaveTopo wave_topology(const int32_t *par, int n) {
    const int lane = lane_id();
    return wave_topology_p(lane < n ? par[lane] : -1, n);
}

// Topology and cumulative log-decay in one doubling pass. Lane i starts from its own
// log-gate lg; each round adds the sum held by the lane its pointer names, then jumps
// the pointer. After the last round, `L` is the sum of lg over every node on the
// root-to-i path. The summation order is a fixed binary tree over the path (the same
// on every call), so the result is deterministic.
struct WaveTopoL {
    uint64_t mask;
    int depth;
    int bad;
    float L;
};

__device__ __forceinline__ WaveTopoL wave_topology_cumlog(int p_loaded, float lg, int n) {
    const int lane = lane_id();
    const int p = lane < n ? p_loaded : -1;
    const bool bad_lane = lane < n && (p < -1 || p >= lane);
    WaveTopoL t;
    t.bad = __any(bad_lane) ? BOLE_TREE_BAD_PARENT : BOLE_TREE_OK;
    const bool live = lane < n && !t.bad;
    uint64_t m = live ? (1ull << lane) : 0ull;
    float acc = live ? lg : 0.f;
    int anc = live ? p : -1;
    for (int r = 0; r < 6 && __any(anc >= 0); ++r) {
        const int src = anc < 0 ? lane : anc;
        const uint64_t m_up = shfl_u64(m, src);
        const float acc_up = __shfl(acc, src, 64);
        const int anc_up = __shfl(anc, src, 64);
        if (anc >= 0) {
            m |= m_up;
            acc += acc_up;
            anc = anc_up;
        }
    }
    t.mask = m;
    t.depth = __popcll(m);
    t.L = acc;
    return t;
}

template <typename T>
__device__ __forceinline__ float to_f32(T x) {
    return static_cast<float>(x);
}

}  // namespace bole
