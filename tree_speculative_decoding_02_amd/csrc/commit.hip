// commit.hip - in-place commit of each tree's accepted path into the committed state.
//
// This is the restore step of the Bole summary page, section 2 ("Token-Level Factor
// Encoding"): after verification, only the accepted path's state is rebuilt, from the
// per-node factors, on top of H_0. For path p_1..p_L of tree b and every head:
//     H_0 <- S_{p_L} ... S_{p_1} H_0 + sum_m (S_{p_L} ... S_{p_{m+1}}) k_{p_m} v_{p_m}^T
// Each thread keeps a slice of H_0 in registers and applies the L rank-one steps
// H <- S_m H + k_m v_m^T in path order, so H_0 is read once and written once. The path
// factors are staged in LDS (as fp32) in chunks of 16 nodes.
//
// One 256-thread workgroup per (sequence, head). The kernel is a stream: its cost is
// the state's round trip through HBM plus a short chain of dependent loads, so it is
// built for occupancy (few registers, little LDS) and a short chain:
//   1. tree offsets and path length (scalar loads);
//   2. the thread's state slice, every parent of the tree and the path indices, all
//      issued together;
//   3. wavefront 0 validates everything with cross-lane operations on what it already
//      holds: tree size, parent links (-1 <= parent[i] < i), path length in
//      [0, max_path], path indices inside the tree, each node the child of the previous
//      one, the first a root;
//   4. the path's factors are staged, the state is updated and stored.
// A bad tree keeps its state. A tree with L = 0 costs no state traffic.
#include "bole_device.h"
#include "launch.h"

namespace bole {

constexpr int kCommitThreads = 256;
constexpr int kPathChunk = 16;   // path nodes staged in LDS at a time
constexpr int kRegFloats = 32;   // state floats held per thread per pass

template <typename TF, bool VEC, int W>
__global__ __launch_bounds__(kCommitThreads) void commit_kernel(
    float *__restrict__ H0, const TF *__restrict__ k, const TF *__restrict__ v,
    const float *__restrict__ gate, const int32_t *__restrict__ parent,
    const int32_t *__restrict__ node_offsets, const int32_t *__restrict__ accepted_idx,
    const int32_t *__restrict__ accepted_len, int32_t *__restrict__ path_nodes,
    int32_t *__restrict__ tree_status, const int32_t *gate_check, int H, int DK, int DV, int T,
    int max_path, int max_n) {
    __shared__ int s_row[kMaxTree];         // packed row of each path node
    __shared__ float s_a[kMaxTree];         // scalar gate of each path node
    __shared__ int s_len;
    extern __shared__ float s_f[];          // [kPathChunk][(VEC ? 2 : 1) * DK + DV] staged factors
    const int unit = blockIdx.x;
    const int b = unit / H, h = unit - b * H;
    const int tid = threadIdx.x;

    const int FW = (VEC ? 2 : 1) * DK + DV;   // staged floats per path node
    const int GPR = DV / W;                    // W-wide groups per state row
    const int G = DK * GPR;                    // groups per state
    constexpr int PER = kRegFloats / W;        // groups per thread per pass
    float *Hu = H0 + (size_t)unit * DK * DV;

    // ---- 1, 2: offsets and length, then everything that depends only on them
    const TreeRange tr = tree_range(node_offsets, b, T, max_n);
    const int len_raw = accepted_len[b];
    const bool likely = tr.status == BOLE_TREE_OK && len_raw > 0 && len_raw <= max_path &&
                        len_raw <= tr.n;
    float reg[PER][W];
    if (likely) {
#pragma unroll
        for (int s = 0; s < PER; ++s) {
            const int g = s * kCommitThreads + tid;
            if (g < G) {
                if constexpr (W == 4) {
                    const float4 t = *reinterpret_cast<const float4 *>(Hu + (size_t)g * 4);
                    reg[s][0] = t.x; reg[s][1] = t.y; reg[s][2] = t.z; reg[s][3] = t.w;
                } else {
                    reg[s][0] = Hu[g];
                }
            }
        }
    }

    // ---- 3: validation by wavefront 0, lane = tree node / path position
    if (tid < 64) {
        int st = tr.status;
        int len = 0, x = -1;
        if (st == BOLE_TREE_OK && tr.n > 0) {
            const int n = tr.n;
            const int p = tid < n ? parent[tr.lo + tid] : -1;
            const bool len_ok = len_raw >= 0 && len_raw <= max_path;
            const int xr = (len_ok && tid < len_raw) ? accepted_idx[(size_t)b * max_path + tid] : -1;
            if (__any(tid < n && (p < -1 || p >= tid))) {
                st = BOLE_TREE_BAD_PARENT;
            } else if (!len_ok) {
                st = BOLE_TREE_BAD_PATH;
            } else {
                len = len_raw;
                x = xr;
                // parent of node x (held by lane x) and the previous path node
                const int px = __shfl(p, (x >= 0 && x < n) ? x : 0, 64);
                const int prev_raw = __shfl(x, tid > 0 ? tid - 1 : 0, 64);
                const int prev = tid == 0 ? -1 : prev_raw;
                const bool bad = tid < len && (x < 0 || x >= n || px != prev);
                if (__any(bad)) st = BOLE_TREE_BAD_PATH;
            }
        } else if (st == BOLE_TREE_OK) {
            // empty tree: only a zero-length path is valid
            if (len_raw != 0) st = BOLE_TREE_BAD_PATH;
        }
        if (st == BOLE_TREE_OK && gate_check && gate_check[b] == BOLE_TREE_BAD_GATE)
            st = BOLE_TREE_BAD_GATE;
        const bool ok = st == BOLE_TREE_OK;
        const int row = (ok && tid < len) ? tr.lo + x : -1;
        s_row[tid] = row;
        if (!VEC) s_a[tid] = row >= 0 ? gate[(size_t)row * H + h] : 1.f;
        if (tid == 0) s_len = ok ? len : 0;
        if (h == 0) {
            if (tid == 0 && tree_status) tree_status[b] = st;
            if (path_nodes && tid < max_path) path_nodes[(size_t)b * max_path + tid] = row;
        }
    }
    __syncthreads();
    const int len = s_len;
    if (len == 0) return;

    // ---- 4: stage factors, update, store
    for (int g0 = 0; g0 < G; g0 += kCommitThreads * PER) {
        if (g0 > 0) {
#pragma unroll
            for (int s = 0; s < PER; ++s) {
                const int g = g0 + s * kCommitThreads + tid;
                if (g < G) {
                    if constexpr (W == 4) {
                        const float4 t = *reinterpret_cast<const float4 *>(Hu + (size_t)g * 4);
                        reg[s][0] = t.x; reg[s][1] = t.y; reg[s][2] = t.z; reg[s][3] = t.w;
                    } else {
                        reg[s][0] = Hu[g];
                    }
                }
            }
        }
        // state row and first column of each group this thread holds (fixed for the pass)
        int rr[PER], cc[PER];
#pragma unroll
        for (int s = 0; s < PER; ++s) {
            const int g = g0 + s * kCommitThreads + tid;
            rr[s] = g / GPR;
            cc[s] = (g - rr[s] * GPR) * W;
        }
        for (int m0 = 0; m0 < len; m0 += kPathChunk) {
            const int mc = min(kPathChunk, len - m0);
            __syncthreads();
            for (int idx = tid; idx < mc * FW; idx += kCommitThreads) {
                const int mm = idx / FW, f = idx - mm * FW;
                const size_t row = (size_t)s_row[m0 + mm];
                float val;
                if (f < DK)
                    val = to_f32(k[(row * H + h) * DK + f]);
                else if (VEC && f < 2 * DK)
                    val = gate[(row * H + h) * DK + (f - DK)];
                else
                    val = to_f32(v[(row * H + h) * DV + (f - (VEC ? 2 : 1) * DK)]);
                s_f[idx] = val;
            }
            __syncthreads();
            for (int mm = 0; mm < mc; ++mm) {
                const float *fk = s_f + mm * FW;
                const float *fg = fk + DK;
                const float *fv = fk + (VEC ? 2 : 1) * DK;
                const float a = VEC ? 0.f : s_a[m0 + mm];
#pragma unroll
                for (int s = 0; s < PER; ++s) {
                    const int g = g0 + s * kCommitThreads + tid;
                    if (g < G) {
                        const float kr = fk[rr[s]];
                        const float sr = VEC ? fg[rr[s]] : a;
#pragma unroll
                        for (int e = 0; e < W; ++e) reg[s][e] = sr * reg[s][e] + kr * fv[cc[s] + e];
                    }
                }
            }
        }
#pragma unroll
        for (int s = 0; s < PER; ++s) {
            const int g = g0 + s * kCommitThreads + tid;
            if (g < G) {
                if constexpr (W == 4) {
                    *reinterpret_cast<float4 *>(Hu + (size_t)g * 4) =
                        make_float4(reg[s][0], reg[s][1], reg[s][2], reg[s][3]);
                } else {
                    Hu[g] = reg[s][0];
                }
            }
        }
    }
}

// Streaming commit for the common shapes: d_v/4 a power of two that divides 256 (so a
// thread's state rows are r0 + 16s-style strides and its columns are fixed), 16-byte
// factor rows. Two dependent rounds of memory instead of three:
//   round 1: tree offsets and path length (scalar), and the path indices the thread's
//            factor chunks and validation need (per lane);
//   round 2: the state slice (non-temporal), the path's factor rows as 16-byte chunks,
//            the tree's parent links and the path's scalar gates, all at once.
// Validation then runs on values already in registers, the factors go to LDS as fp32,
// and the state is updated in registers and stored (non-temporal). Up to 16 path nodes
// are staged per round; longer paths stage the rest afterwards.
constexpr int kStageNodes = 16;
constexpr unsigned kCommitTargetBlocks = 1024;  // small batches split states to about this many
typedef float f32x4v __attribute__((ext_vector_type(4)));

// Layer blockIdx.y of the table (its H0, k, v, gate); the layers share trees and paths,
// and layer 0 writes the per-tree outputs.
template <typename TF, bool VEC, bool SLICED>
__global__ __launch_bounds__(kCommitThreads) void commit_stream_kernel(
    const LayerTable lt, const int32_t *__restrict__ parent,
    const int32_t *__restrict__ node_offsets, const int32_t *__restrict__ accepted_idx,
    const int32_t *__restrict__ accepted_len, int32_t *__restrict__ path_nodes,
    int32_t *__restrict__ tree_status, const int32_t *gate_check, int H, int DK, int DV, int T,
    int max_path, int max_n, int gpr_log2, int slices, int slice_groups) {
    const bole_layer_t &ly = lt.l[blockIdx.y];
    float *const H0 = ly.H0;
    const TF *const k = static_cast<const TF *>(ly.k);
    const TF *const v = static_cast<const TF *>(ly.v);
    const float *const gate = ly.gate;
    constexpr int E = 16 / sizeof(TF);   // factor elements per 16-byte chunk
    constexpr int PER = kRegFloats / 4;  // float4 state groups per thread per pass
    __shared__ int s_row[kMaxTree];
    __shared__ float s_a[kMaxTree];
    __shared__ int s_len;
    extern __shared__ __attribute__((aligned(16))) float s_f[];  // [kStageNodes][FW]: k, (gate), v rows
    // workgroup = (unit, slice): the slice is a run of slice_groups float4 groups of the
    // unit's state (whole state when slices == 1)
    const int unit = SLICED ? (int)blockIdx.x / slices : (int)blockIdx.x;
    const int slice = SLICED ? (int)blockIdx.x - unit * slices : 0;
    const int b = unit / H, h = unit - b * H;
    const int tid = threadIdx.x;
    const int FW = (VEC ? 2 : 1) * DK + DV;
    const int CK = DK / E, CG = VEC ? DK / 4 : 0, CV = DV / E;
    const int CPN = CK + CG + CV;        // chunks per path node
    // this slice: groups gbeg .. gbeg + G - 1 of the state, i.e. rows from row0 on
    const int gbeg = SLICED ? slice * slice_groups : 0;
    const int G = SLICED ? min(DK * DV / 4 - gbeg, slice_groups) : DK * DV / 4;
    const int row0 = SLICED ? gbeg >> gpr_log2 : 0;
    float *Hu = H0 + (size_t)unit * DK * DV + (size_t)gbeg * 4;

    // ---- round 1
    const TreeRange tr = tree_range(node_offsets, b, T, max_n);
    const int len_raw = accepted_len[b];
    const int m0 = tid / CPN, m1 = (tid + kCommitThreads) / CPN;  // nodes of my two chunks
    const int32_t *acc_b = accepted_idx + (size_t)b * max_path;
    const int x0 = m0 < max_path ? acc_b[m0] : 0;
    const int x1 = m1 < max_path ? acc_b[m1] : 0;
    const int xl = (tid < 64 && tid < max_path) ? acc_b[tid] : -1;

    // ---- round 2
    const bool likely = tr.status == BOLE_TREE_OK && len_raw > 0 && len_raw <= max_path &&
                        len_raw <= tr.n;
    const int n = tr.n;
    f32x4v reg[PER];
    const int rs = kCommitThreads >> gpr_log2;             // state rows between groups
    const int r0 = tid >> gpr_log2;                        // row of group 0 (of a pass)
    const int cc = (tid & ((1 << gpr_log2) - 1)) * 4;      // first column (fixed)
    if (likely) {
#pragma unroll
        for (int s = 0; s < PER; ++s) {
            const int g = s * kCommitThreads + tid;
            if (g < G) reg[s] = __builtin_nontemporal_load(reinterpret_cast<const f32x4v *>(Hu) + g);
        }
    }
    // factor chunks of the first S1 path nodes, two chunks per thread at most (clamped
    // rows: validated below); later nodes are staged kStageNodes at a time
    const int S1 = min(kStageNodes, 2 * kCommitThreads / CPN);
    const int L0 = likely ? min(len_raw, S1) : 0;
    auto chunk_src = [&](int c, int x) -> const void * {
        const int m = c / CPN, part = c - m * CPN;
        (void)m;
        const size_t row = (size_t)(tr.lo + min(max(x, 0), n - 1)) * H + h;
        if (part < CK) return k + row * DK + part * E;
        if (VEC && part < CK + CG) return gate + row * DK + (part - CK) * 4;
        return v + row * DV + (part - CK - CG) * E;
    };
    uint4 raw0 = {0, 0, 0, 0}, raw1 = {0, 0, 0, 0};
    const int c0 = tid, c1 = tid + kCommitThreads;
    if (c0 < L0 * CPN) raw0 = *reinterpret_cast<const uint4 *>(chunk_src(c0, x0));
    if (c1 < L0 * CPN) raw1 = *reinterpret_cast<const uint4 *>(chunk_src(c1, x1));

    // validation by wavefront 0 (lane = tree node / path position)
    if (tid < 64) {
        int st = tr.status;
        int len = 0, x = -1;
        float a = 1.f;
        if (st == BOLE_TREE_OK && n > 0) {
            const int p = tid < n ? parent[tr.lo + tid] : -1;
            const bool len_ok = len_raw >= 0 && len_raw <= max_path;
            const int xr = (len_ok && tid < len_raw) ? xl : -1;
            if (!VEC && len_ok && tid < len_raw)
                a = gate[(size_t)(tr.lo + min(max(xr, 0), n - 1)) * H + h];
            if (__any(tid < n && (p < -1 || p >= tid))) {
                st = BOLE_TREE_BAD_PARENT;
            } else if (!len_ok) {
                st = BOLE_TREE_BAD_PATH;
            } else {
                len = len_raw;
                x = xr;
                const int px = __shfl(p, (x >= 0 && x < n) ? x : 0, 64);
                const int prev_raw = __shfl(x, tid > 0 ? tid - 1 : 0, 64);
                const int prev = tid == 0 ? -1 : prev_raw;
                const bool bad = tid < len && (x < 0 || x >= n || px != prev);
                if (__any(bad)) st = BOLE_TREE_BAD_PATH;
            }
        } else if (st == BOLE_TREE_OK) {
            if (len_raw != 0) st = BOLE_TREE_BAD_PATH;  // empty tree: only L = 0 is valid
        }
        // a gate outside its domain (BOLE_FLAG_VALIDATE_GATES): the sequence keeps its
        // state. The workgroup writing tree_status writes the same decision it reads here,
        // so every workgroup of the tree decides alike whichever value it reads.
        if (st == BOLE_TREE_OK && gate_check && gate_check[b] == BOLE_TREE_BAD_GATE)
            st = BOLE_TREE_BAD_GATE;
        const bool ok = st == BOLE_TREE_OK;
        const int row = (ok && tid < len) ? tr.lo + x : -1;
        s_row[tid] = row;
        s_a[tid] = a;
        if (tid == 0) s_len = ok ? len : 0;
        if (h == 0 && slice == 0 && blockIdx.y == 0) {
            if (tid == 0 && tree_status) tree_status[b] = st;
            if (path_nodes && tid < max_path) path_nodes[(size_t)b * max_path + tid] = row;
        }
    }
    // factors -> LDS as fp32
    auto put = [&](int c, const uint4 &raw) {
        const int m = c / CPN, part = c - m * CPN;
        float *dst = s_f + m * FW;
        if (part < CK) {
            dst += part * E;
        } else if (VEC && part < CK + CG) {
            dst += DK + (part - CK) * 4;
            *reinterpret_cast<uint4 *>(dst) = raw;
            return;
        } else {
            dst += (VEC ? 2 : 1) * DK + (part - CK - CG) * E;
        }
        if (E == 8) {
            const __bf16 *e = reinterpret_cast<const __bf16 *>(&raw);
            *reinterpret_cast<float4 *>(dst) = make_float4(to_f32(e[0]), to_f32(e[1]), to_f32(e[2]), to_f32(e[3]));
            *reinterpret_cast<float4 *>(dst + 4) = make_float4(to_f32(e[4]), to_f32(e[5]), to_f32(e[6]), to_f32(e[7]));
        } else {
            *reinterpret_cast<uint4 *>(dst) = raw;
        }
    };
    if (c0 < L0 * CPN) put(c0, raw0);
    if (c1 < L0 * CPN) put(c1, raw1);
    __syncthreads();
    const int len = s_len;
    if (len == 0) return;

    for (int g0 = 0; g0 < G; g0 += kCommitThreads * PER) {
        const int rbase = (g0 >> gpr_log2) + r0;
        if (g0 > 0) {
#pragma unroll
            for (int s = 0; s < PER; ++s) {
                const int g = g0 + s * kCommitThreads + tid;
                if (g < G) reg[s] = __builtin_nontemporal_load(reinterpret_cast<const f32x4v *>(Hu) + g);
            }
        }
        for (int m0s = 0; m0s < len;) {
            const int mc = m0s == 0 ? min(S1, len) : min(kStageNodes, len - m0s);
            if (m0s > 0 || g0 > 0) {
                // stage path nodes m0s .. m0s+mc-1 (the first group is staged above)
                __syncthreads();
                for (int c = tid; c < mc * CPN; c += kCommitThreads) {
                    const int m = c / CPN, part = c - m * CPN;
                    const size_t row = (size_t)s_row[m0s + m] * H + h;
                    const void *src;
                    if (part < CK) src = k + row * DK + part * E;
                    else if (VEC && part < CK + CG) src = gate + row * DK + (part - CK) * 4;
                    else src = v + row * DV + (part - CK - CG) * E;
                    put(c, *reinterpret_cast<const uint4 *>(src));
                }
                __syncthreads();
            }
            for (int mm = 0; mm < mc; ++mm) {
                const float *fk = s_f + mm * FW + row0;  // k and gate rows of this slice
                const float *fg = fk + DK;
                const float4 vv = *reinterpret_cast<const float4 *>(s_f + mm * FW + (VEC ? 2 : 1) * DK + cc);
                const float a = s_a[m0s + mm];
#pragma unroll
                for (int s = 0; s < PER; ++s) {
                    const int r = rbase + s * rs;
                    if (g0 + s * kCommitThreads + tid < G) {
                        const float kr = fk[r];
                        const float sr = VEC ? fg[r] : a;
                        reg[s].x = sr * reg[s].x + kr * vv.x;
                        reg[s].y = sr * reg[s].y + kr * vv.y;
                        reg[s].z = sr * reg[s].z + kr * vv.z;
                        reg[s].w = sr * reg[s].w + kr * vv.w;
                    }
                }
            }
            m0s += mc;
        }
#pragma unroll
        for (int s = 0; s < PER; ++s) {
            const int g = g0 + s * kCommitThreads + tid;
            if (g < G) __builtin_nontemporal_store(reg[s], reinterpret_cast<f32x4v *>(Hu) + g);
        }
    }
}

template <typename TF, bool VEC>
static void launch_w(const bole_layer_t *layers, int nl, const int32_t *parent,
                     const int32_t *node_offsets, const int32_t *accepted_idx,
                     const int32_t *accepted_len, const bole_dims_t &d, int32_t *path_nodes,
                     int32_t *tree_status, const int32_t *gate_check, hipStream_t stream) {
    const dim3 block(kCommitThreads);
    // streaming kernel: d_v/4 a power of two dividing the block, 16-byte state and factor
    // rows in every layer
    const int gpr = d.d_v / 4;
    constexpr int E = 16 / sizeof(TF);
    bool vec4 = d.d_v % 4 == 0, aligned = true;
    for (int l = 0; l < nl; ++l) {
        vec4 = vec4 && reinterpret_cast<uintptr_t>(layers[l].H0) % 16 == 0;
        const uintptr_t fa = reinterpret_cast<uintptr_t>(layers[l].k) |
                             reinterpret_cast<uintptr_t>(layers[l].v) |
                             (VEC ? reinterpret_cast<uintptr_t>(layers[l].gate) : 0);
        aligned = aligned && fa % 16 == 0;
    }
    if (vec4 && aligned && gpr > 0 && (gpr & (gpr - 1)) == 0 && kCommitThreads % gpr == 0 &&
        d.d_k % E == 0 && d.d_v % E == 0) {
        const size_t slds = sizeof(float) * kStageNodes * ((VEC ? 2 : 1) * d.d_k + d.d_v);
        // state slices per unit: one pass per workgroup, and about kCommitTargetBlocks
        // workgroups per layer when the batch is small
        const unsigned U = (unsigned)d.batch * (unsigned)d.heads;
        const int G = d.d_k * d.d_v / 4, per_pass = kCommitThreads * kRegFloats / 4;
        int slices = (G + per_pass - 1) / per_pass;
        const int want = (int)((kCommitTargetBlocks + U - 1) / U);
        slices = max(slices, min(want, G / kCommitThreads));
        int sg = (G + slices - 1) / slices;
        sg = (sg + kCommitThreads - 1) / kCommitThreads * kCommitThreads;
        slices = (G + sg - 1) / sg;
        LayerTable lt = {};
        for (int l = 0; l < nl; ++l) lt.l[l] = layers[l];
        auto kern = slices > 1 ? commit_stream_kernel<TF, VEC, true> : commit_stream_kernel<TF, VEC, false>;
        kern<<<dim3(U * (unsigned)slices, (unsigned)nl), block, slds, stream>>>(
            lt, parent, node_offsets, accepted_idx, accepted_len, path_nodes, tree_status,
            gate_check, d.heads, d.d_k, d.d_v, d.total_nodes, d.max_path, max_tree_nodes(d.flags),
            __builtin_ctz((unsigned)gpr), slices, sg);
        return;
    }
    // any other shape or alignment: one launch per layer
    const dim3 grid((unsigned)d.batch * (unsigned)d.heads);
    const size_t lds = sizeof(float) * kPathChunk * ((VEC ? 2 : 1) * d.d_k + d.d_v);
    for (int l = 0; l < nl; ++l) {
        const bole_layer_t &y = layers[l];
        const TF *k = static_cast<const TF *>(y.k), *v = static_cast<const TF *>(y.v);
        int32_t *pn = l == 0 ? path_nodes : nullptr, *ts = l == 0 ? tree_status : nullptr;
        if (d.d_v % 4 == 0 && reinterpret_cast<uintptr_t>(y.H0) % 16 == 0)
            commit_kernel<TF, VEC, 4><<<grid, block, lds, stream>>>(
                y.H0, k, v, y.gate, parent, node_offsets, accepted_idx, accepted_len, pn, ts,
                gate_check, d.heads, d.d_k, d.d_v, d.total_nodes, d.max_path, max_tree_nodes(d.flags));
        else
            commit_kernel<TF, VEC, 1><<<grid, block, lds, stream>>>(
                y.H0, k, v, y.gate, parent, node_offsets, accepted_idx, accepted_len, pn, ts,
                gate_check, d.heads, d.d_k, d.d_v, d.total_nodes, d.max_path, max_tree_nodes(d.flags));
    }
}

hipError_t launch_commit(const bole_layer_t *layers, int nl, const int32_t *parent,
                         const int32_t *node_offsets, const int32_t *accepted_idx,
                         const int32_t *accepted_len, const bole_dims_t &d, int32_t *path_nodes,
                         int32_t *tree_status, const int32_t *gate_check, hipStream_t stream) {
    const bool vec = d.gate_kind == BOLE_GATE_VECTOR;
    if (d.factor_dtype == BOLE_DTYPE_F32) {
        if (vec) launch_w<float, true>(layers, nl, parent, node_offsets, accepted_idx, accepted_len, d, path_nodes, tree_status, gate_check, stream);
        else launch_w<float, false>(layers, nl, parent, node_offsets, accepted_idx, accepted_len, d, path_nodes, tree_status, gate_check, stream);
    } else {
        if (vec) launch_w<__bf16, true>(layers, nl, parent, node_offsets, accepted_idx, accepted_len, d, path_nodes, tree_status, gate_check, stream);
        else launch_w<__bf16, false>(layers, nl, parent, node_offsets, accepted_idx, accepted_len, d, path_nodes, tree_status, gate_check, stream);
    }
    return hipGetLastError();
}

}  // namespace bole
