// verify_naive.hip - the naive serial walk that the closed form replaces (Bole summary
// page, section 1: without the closed form, a tree is verified by walking it node by
// node and keeping one state per node). Kept as the baseline the closed form is
// measured against: its time, and the transient memory of the states it materialises.
//
// One workgroup per (sequence, head) walks the tree in index order (a parent always
// precedes its children):
//     H_i = S_i H_parent(i) + k_i v_i^T   (H_parent = H_0 for a root),   out_i = H_i^T q_i,
// writing every H_i to the caller's states buffer [T][H][d_k][d_v]. Thread t owns state
// column t % d_v and rows t / d_v, t / d_v + RS, ... (RS = threads / d_v), the same
// entries for every node, so it only ever reads back states it wrote itself; the output
// dot products are summed over the RS row sets in LDS.
#include "bole_device.h"
#include "launch.h"

namespace bole {

template <typename TF, bool VEC>
__global__ __launch_bounds__(256) void verify_naive_kernel(
    const float *__restrict__ H0, const TF *__restrict__ q, const TF *__restrict__ k,
    const TF *__restrict__ v, const float *__restrict__ gate,
    const int32_t *__restrict__ parent, const int32_t *__restrict__ node_offsets,
    float *__restrict__ out, float *__restrict__ states, int32_t *__restrict__ tree_status,
    int H, int DK, int DV, int T, int max_n, int RS) {
    extern __shared__ float s_part[];  // [RS][DV] partial output sums
    __shared__ int s_bad;
    const int unit = blockIdx.x;
    const int b = unit / H, h = unit - b * H;
    const int tid = threadIdx.x;
    const int c = tid % DV, rsl = tid / DV;
    const bool writer = tree_status != nullptr && h == 0 && tid == 0;

    const TreeRange tr = tree_range(node_offsets, b, T, max_n);
    if (tr.status != BOLE_TREE_OK) {
        if (writer) tree_status[b] = tr.status;
        return;
    }
    const int lo = tr.lo, n = tr.n;
    if (n == 0) {
        if (writer) tree_status[b] = BOLE_TREE_OK;
        return;
    }
    // parent links: -1 <= parent[i] < i, checked before anything is written
    if (tid < 64) {
        const int p = tid < n ? parent[lo + tid] : -1;
        const bool bad = __any(tid < n && (p < -1 || p >= tid));
        if (tid == 0) s_bad = bad ? BOLE_TREE_BAD_PARENT : BOLE_TREE_OK;
    }
    __syncthreads();
    if (writer) tree_status[b] = s_bad;
    if (s_bad != BOLE_TREE_OK) {
        for (int e = tid; e < n * DV; e += blockDim.x)
            out[((size_t)(lo + e / DV) * H + h) * DV + (e % DV)] = __builtin_nanf("");
        return;
    }

    const size_t SS = (size_t)DK * DV;  // floats per state
    for (int i = 0; i < n; ++i) {
        const int p = parent[lo + i];
        const size_t row = (size_t)(lo + i) * H + h;
        const float *src = p < 0 ? H0 + (size_t)unit * SS : states + ((size_t)(lo + p) * H + h) * SS;
        float *dst = states + row * SS;
        const float a = VEC ? 0.f : gate[row];
        const float vc = to_f32(v[row * DV + c]);
        float part = 0.f;
        if (rsl < RS) {
            for (int r = rsl; r < DK; r += RS) {
                const float s = VEC ? gate[row * DK + r] : a;
                const float x = s * src[(size_t)r * DV + c] + to_f32(k[row * DK + r]) * vc;
                dst[(size_t)r * DV + c] = x;
                part += x * to_f32(q[row * DK + r]);
            }
            s_part[rsl * DV + c] = part;
        }
        __syncthreads();
        if (tid < DV) {
            float o = 0.f;
            for (int j = 0; j < RS; ++j) o += s_part[j * DV + tid];
            out[row * DV + tid] = o;
        }
        __syncthreads();
    }
}

template <typename TF, bool VEC>
static void launch_naive_t(const float *H0, const void *q, const void *k, const void *v,
                           const float *gate, const int32_t *parent, const int32_t *node_offsets,
                           float *out, float *states, const bole_dims_t &d,
                           int32_t *tree_status, hipStream_t stream) {
    const int RS = d.d_v >= 256 ? 1 : 256 / d.d_v;  // row sets per column
    const unsigned threads = (unsigned)(RS * d.d_v);
    const unsigned U = (unsigned)d.batch * (unsigned)d.heads;
    verify_naive_kernel<TF, VEC><<<dim3(U), dim3(threads), sizeof(float) * RS * d.d_v, stream>>>(
        H0, static_cast<const TF *>(q), static_cast<const TF *>(k), static_cast<const TF *>(v),
        gate, parent, node_offsets, out, states, tree_status, d.heads, d.d_k, d.d_v,
        d.total_nodes, max_tree_nodes(d.flags), RS);
}

hipError_t launch_verify_naive(const float *H0, const void *q, const void *k, const void *v,
                               const float *gate, const int32_t *parent,
                               const int32_t *node_offsets, float *out, float *states,
                               const bole_dims_t &d, int32_t *tree_status, hipStream_t stream) {
    const bool vec = d.gate_kind == BOLE_GATE_VECTOR;
    if (d.factor_dtype == BOLE_DTYPE_F32) {
        if (vec) launch_naive_t<float, true>(H0, q, k, v, gate, parent, node_offsets, out, states, d, tree_status, stream);
        else launch_naive_t<float, false>(H0, q, k, v, gate, parent, node_offsets, out, states, d, tree_status, stream);
    } else {
        if (vec) launch_naive_t<__bf16, true>(H0, q, k, v, gate, parent, node_offsets, out, states, d, tree_status, stream);
        else launch_naive_t<__bf16, false>(H0, q, k, v, gate, parent, node_offsets, out, states, d, tree_status, stream);
    }
    return hipGetLastError();
}

}  // namespace bole
