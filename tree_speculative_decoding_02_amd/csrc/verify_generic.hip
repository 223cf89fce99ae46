// verify_generic.hip - plain vector-ALU tree verification, fp32 arithmetic.
//
// It evaluates the closed form of the Bole summary page, section 1 ("Tree-Structured
// Closed Form"), for any supported shape:
//     o_i = D_i (H_0^T q_i) + sum_{j on path(i)} D_{j->i} (q_i . k_j) v_j
// channel by channel for vector gates. All nodes are done in parallel; no per-node
// state is formed. It covers fp32 factors, vector gates, and any d_k/d_v up to 256 (a
// vector gate's per-channel cumulative log-decay takes 64 d_k floats of LDS: 64 KB at
// d_k = 256, within gfx950's 160 KB). The matrix-core kernel in verify_mfma.hip serves the
// bf16 scalar-gate shapes that matter for throughput. This one is the fp32-accurate
// baseline and the fallback. With fp32 factors it accumulates in fp64 (dot products, the
// H_0 term, the sum over the path, and the cumulative log-decays summed along each path):
// a query and key can nearly cancel in their dot product (q.k a thousandth of |q||k|), and
// fp32 accumulation then errs by about 1e-5 of the output row; fp32 inputs are exact in
// fp64. bf16 factors accumulate in fp32.
//
// One 256-thread workgroup per (sequence, head):
//   1. wavefront 0 builds the tree topology (ancestor masks) and, for scalar gates,
//      the root-first cumulative log-decay L_i; for vector gates every thread fills
//      L_i[c] in LDS;
//   2. pair weights W_ij = (q_i . k_j) exp(L_i - L_j) for every ancestor-or-self j
//      (vector: sum_c q_i[c] k_j[c] exp(L_i[c] - L_j[c])), zero elsewhere, into LDS;
//   3. each output element: exp(L_i) sum_r H0[r][c] q_i[r] + sum_j W_ij v_j[c].
#include <type_traits>

#include "bole_device.h"
#include "launch.h"

namespace bole {

__device__ __forceinline__ float gexp(float x) { return expf(x); }
__device__ __forceinline__ double gexp(double x) { return exp(x); }
__device__ __forceinline__ float glog(float x) { return logf(x); }
__device__ __forceinline__ double glog(double x) { return log(x); }

template <typename TF, bool VEC>
__global__ __launch_bounds__(256) void verify_generic_kernel(
    const float *__restrict__ H0, const TF *__restrict__ q, const TF *__restrict__ k,
    const TF *__restrict__ v, const float *__restrict__ gate, const int32_t *__restrict__ parent,
    const int32_t *__restrict__ node_offsets, float *__restrict__ out,
    int32_t *__restrict__ tree_status, int H, int DK, int DV, int T, int max_n) {
    // accumulation type: fp64 for fp32 factors, fp32 for bf16
    typedef typename std::conditional<std::is_same<TF, float>::value, double, float>::type A;
    __shared__ uint64_t s_mask[kMaxTree];
    __shared__ A s_L[kMaxTree];
    __shared__ float s_W[kMaxTree][kMaxTree + 1];
    __shared__ int s_bad;
    extern __shared__ __align__(16) unsigned char s_dyn[];
    A *const s_Lv = reinterpret_cast<A *>(s_dyn);  // VEC: [n][DK] cumulative log-decay per channel

    const int unit = blockIdx.x;
    const int b = unit / H, h = unit - b * H;
    const int tid = threadIdx.x;
    const TreeRange tr = tree_range(node_offsets, b, T, max_n);
    if (tr.status != BOLE_TREE_OK) {
        if (h == 0 && tid == 0 && tree_status) tree_status[b] = tr.status;
        return;
    }
    const int lo = tr.lo, n = tr.n;
    if (tid < 64) {
        const int p_raw = tid < n ? parent[lo + tid] : -1;
        const float lg =
            (!VEC && tid < n) ? logf(gate[(size_t)(lo + tid) * H + h]) : 0.f;
        const WaveTopoL t = wave_topology_cumlog(p_raw, lg, n);
        if (tid == 0) s_bad = t.bad;
        s_mask[tid] = t.mask;
        A L = t.L;
        if (sizeof(A) == 8 && !VEC) {
            // fp64: log-gates summed along the node's path, root first
            L = 0;
            for (uint64_t mm = t.bad ? 0ull : t.mask; mm; mm &= mm - 1)
                L += glog((A)gate[(size_t)(lo + __ffsll((unsigned long long)mm) - 1) * H + h]);
        }
        s_L[tid] = L;
    }
    __syncthreads();
    const int bad = s_bad;
    if (h == 0 && tid == 0 && tree_status) tree_status[b] = bad;
    const size_t rq = (size_t)H * DK, rv = (size_t)H * DV;
    if (bad) {
        for (int idx = tid; idx < n * DV; idx += 256) {
            const int i = idx / DV, c = idx - i * DV;
            out[(size_t)(lo + i) * rv + (size_t)h * DV + c] = __builtin_nanf("");
        }
        return;
    }
    if (VEC) {
        for (int idx = tid; idx < n * DK; idx += 256) {
            const int i = idx / DK, c = idx - i * DK;
            const uint64_t m = s_mask[i];
            A L = 0;
            for (int j = 0; j <= i; ++j)
                if ((m >> j) & 1ull) L += glog((A)gate[(size_t)(lo + j) * rq + (size_t)h * DK + c]);
            s_Lv[i * DK + c] = L;
        }
        __syncthreads();
    }
    for (int idx = tid; idx < n * n; idx += 256) {
        const int i = idx / n, j = idx - i * n;
        float w = 0.f;
        if ((s_mask[i] >> j) & 1ull) {
            const TF *qi = q + (size_t)(lo + i) * rq + (size_t)h * DK;
            const TF *kj = k + (size_t)(lo + j) * rq + (size_t)h * DK;
            A acc = 0;
            for (int c = 0; c < DK; ++c) {
                A t = (A)to_f32(qi[c]) * (A)to_f32(kj[c]);
                if (VEC) t *= gexp(s_Lv[i * DK + c] - s_Lv[j * DK + c]);
                acc += t;
            }
            w = (float)(VEC ? acc : acc * gexp(s_L[i] - s_L[j]));
        }
        s_W[i][j] = w;
    }
    __syncthreads();
    const float *H0u = H0 + (size_t)unit * DK * DV;
    for (int idx = tid; idx < n * DV; idx += 256) {
        const int i = idx / DV, c = idx - i * DV;
        const TF *qi = q + (size_t)(lo + i) * rq + (size_t)h * DK;
        A acc = 0;
        for (int r = 0; r < DK; ++r) {
            A qq = (A)to_f32(qi[r]);
            if (VEC) qq *= gexp(s_Lv[i * DK + r]);
            acc += (A)H0u[(size_t)r * DV + c] * qq;
        }
        if (!VEC) acc *= gexp(s_L[i]);
        for (int j = 0; j <= i; ++j)
            acc += (A)s_W[i][j] * (A)to_f32(v[(size_t)(lo + j) * rv + (size_t)h * DV + c]);
        out[(size_t)(lo + i) * rv + (size_t)h * DV + c] = (float)acc;
    }
}

template <typename TF>
static hipError_t launch_typed(const float *H0, const void *q, const void *k, const void *v,
                               const float *gate, const int32_t *parent,
                               const int32_t *node_offsets, float *out, const bole_dims_t &d,
                               int32_t *tree_status, hipStream_t stream) {
    const dim3 grid((unsigned)d.batch * (unsigned)d.heads), block(256);
    const TF *qt = static_cast<const TF *>(q), *kt = static_cast<const TF *>(k),
             *vt = static_cast<const TF *>(v);
    if (d.gate_kind == BOLE_GATE_VECTOR) {
        const size_t lds = (std::is_same<TF, float>::value ? sizeof(double) : sizeof(float)) * kMaxTree * d.d_k;
        if (lds > 65536) {
            // above the default dynamic-LDS limit (fp64 decays at d_k = 256: 128 KB), raised
            // once for this instantiation; 17 KB of static LDS come on top, within 160 KB
            static const hipError_t raised = hipFuncSetAttribute(
                reinterpret_cast<const void *>(&verify_generic_kernel<TF, true>),
                hipFuncAttributeMaxDynamicSharedMemorySize, (int)(sizeof(double) * kMaxTree * 256));
            if (raised != hipSuccess) return raised;
        }
        verify_generic_kernel<TF, true><<<grid, block, lds, stream>>>(
            H0, qt, kt, vt, gate, parent, node_offsets, out, tree_status, d.heads, d.d_k, d.d_v,
            d.total_nodes, max_tree_nodes(d.flags));
    } else {
        verify_generic_kernel<TF, false><<<grid, block, 0, stream>>>(
            H0, qt, kt, vt, gate, parent, node_offsets, out, tree_status, d.heads, d.d_k, d.d_v,
            d.total_nodes, max_tree_nodes(d.flags));
    }
    return hipGetLastError();
}

hipError_t launch_verify_generic(const float *H0, const void *q, const void *k, const void *v,
                                 const float *gate, const int32_t *parent,
                                 const int32_t *node_offsets, float *out, const bole_dims_t &d,
                                 int32_t *tree_status, hipStream_t stream) {
    if (d.factor_dtype == BOLE_DTYPE_F32)
        return launch_typed<float>(H0, q, k, v, gate, parent, node_offsets, out, d, tree_status,
                                   stream);
    return launch_typed<__bf16>(H0, q, k, v, gate, parent, node_offsets, out, d, tree_status,
                                stream);
}

}  // namespace bole
