// tree_accept.hip - which draft nodes the target accepts, and its next token (LLM Primer
// chapter 9 walkthrough, section 9.1: longest agreeing prefix; min(1, p/q) acceptance
// with resampling from the residual (p - q)+).
//
// One workgroup per tree walks down from the verified context, one accepted node at a
// time. Wavefront 0 holds the tree (lane = node: parent, token) and finds the current
// node's children by ballot. Every pass over a vocabulary row uses the whole workgroup;
// every decision is taken once from block-reduced values and is the same in every
// thread.
//  - greedy: the target's argmax (lowest id on ties) picks the child, else is the bonus;
//  - sampling: children in index order, each tested against the residuals left by the
//    rejected ones before it. With rp = p_res * Zp and rq = q_res * Zq unnormalised, x is
//    accepted when u * rq(x) * Zp < rp(x) * Zq. The residuals are never stored: after k
//    rejections rp(y) = max(p(y) A - q(y) C, 0) (a clamp at 0 never releases, so the
//    step-by-step residual has this closed form), with A, C, Zq updated per rejection of
//    x as A <- A / Zp, C <- C / Zp + 1 / Zq, Zq <- Zq - q(x), and Zp the sum of the new
//    rp: one pass over the node's two fp32 rows. The bonus is drawn from rp by inverse
//    CDF. fp64 throughout, products and differences separately rounded.
#include "bole_device.h"
#include "launch.h"

namespace bole {

constexpr int kAcceptThreads = 1024;
constexpr int kAcceptBatch = 16;  // loads in flight per thread in a pass
constexpr int kAcceptWaves = kAcceptThreads / 64;

struct AcceptArgs {
    const float *p_ctx, *p_node, *q_ctx, *q_node, *u_node, *u_bonus;
    const int32_t *parent, *token, *node_offsets;
    int32_t *accepted_idx, *accepted_len, *bonus, *tree_status;
    int B, T, V, max_path, mode;
    bool vec;  // fp32 rows are 16-byte aligned (V % 4 == 0 and aligned bases)
};

// Calls f(y, value) for the elements of an fp32 row this thread owns, in increasing y.
// Loads are issued kAcceptBatch at a time before any is used.
template <typename F>
__device__ __forceinline__ void row_pass(const float *row, int V, bool vec, F f) {
    const int t = threadIdx.x;
    if (vec) {
        typedef float f4 __attribute__((ext_vector_type(4)));
        constexpr int step = 4 * kAcceptThreads;
        for (int y0 = 4 * t; y0 < V; y0 += step * kAcceptBatch) {
            f4 x[kAcceptBatch];
#pragma unroll
            for (int u = 0; u < kAcceptBatch; ++u) {
                const int y = y0 + u * step;
                x[u] = __builtin_nontemporal_load(reinterpret_cast<const f4 *>(row + min(y, V - 4)));
            }
#pragma unroll
            for (int u = 0; u < kAcceptBatch; ++u) {
                const int y = y0 + u * step;
                if (y < V) {
#pragma unroll
                    for (int c = 0; c < 4; ++c) f(y + c, x[u][c]);
                }
            }
        }
    } else {
        for (int y0 = t; y0 < V; y0 += kAcceptThreads * kAcceptBatch) {
            float x[kAcceptBatch];
#pragma unroll
            for (int u = 0; u < kAcceptBatch; ++u)
                x[u] = row[min(y0 + u * kAcceptThreads, V - 1)];
#pragma unroll
            for (int u = 0; u < kAcceptBatch; ++u)
                if (y0 + u * kAcceptThreads < V) f(y0 + u * kAcceptThreads, x[u]);
        }
    }
}

// rp(y) = max(p(y) A - q(y) C, 0), each product and the difference rounded on its own
__device__ __forceinline__ double residual(float p, float q, double A, double C) {
    return fmax(__dsub_rn(__dmul_rn((double)p, A), __dmul_rn((double)q, C)), 0.0);
}

__device__ __forceinline__ double block_sum_d(double x, double *s_red) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
    const int wave = threadIdx.x >> 6;
    __syncthreads();
    if (lane_id() == 0) s_red[wave] = x;
    __syncthreads();
    double t = 0.0;
#pragma unroll
    for (int w = 0; w < kAcceptWaves; ++w) t += s_red[w];
    return t;
}

__global__ __launch_bounds__(kAcceptThreads) void tree_accept_kernel(AcceptArgs a) {
    __shared__ double s_red[kAcceptWaves];
    __shared__ double s_scan[kAcceptThreads];
    __shared__ float s_bv[kAcceptWaves];
    __shared__ int s_bi[kAcceptWaves];
    __shared__ int s_par[kMaxTree], s_tok[kMaxTree];
    __shared__ int s_status, s_n, s_lo, s_pick;
    const int b = blockIdx.x, t = threadIdx.x, lane = lane_id(), wave = t >> 6;
    const int V = a.V;

    // ---- validate the tree (wavefront 0, lane = node)
    if (wave == 0) {
        const TreeRange tr = tree_range(a.node_offsets, b, a.T);
        int st = tr.status;
        const int n = st == BOLE_TREE_OK ? tr.n : 0;
        const int p = lane < n ? a.parent[tr.lo + lane] : -1;
        const int tk = lane < n ? a.token[tr.lo + lane] : 0;
        if (st == BOLE_TREE_OK && __any(lane < n && (p < -1 || p >= lane))) st = BOLE_TREE_BAD_PARENT;
        if (st == BOLE_TREE_OK && __any(lane < n && (tk < 0 || tk >= V))) st = BOLE_TREE_BAD_TOKEN;
        s_par[lane] = lane < n ? p : -2;
        s_tok[lane] = tk;
        if (lane == 0) {
            s_status = st;
            s_n = n;
            s_lo = tr.lo;
        }
    }
    __syncthreads();
    const int st = s_status, n = s_n, lo = s_lo;
    if (st != BOLE_TREE_OK) {
        if (t == 0) {
            if (a.tree_status) a.tree_status[b] = st;
            a.accepted_len[b] = 0;
            a.bonus[b] = -1;
        }
        for (int m = t; m < a.max_path; m += kAcceptThreads) a.accepted_idx[(size_t)b * a.max_path + m] = -1;
        return;
    }

    int cur = -1, len = 0, bonus = -1;
    while (true) {
        const float *prow = cur < 0 ? a.p_ctx + (size_t)b * V : a.p_node + (size_t)(lo + cur) * V;
        // children of cur, in index order (wavefront 0's ballot, shared through LDS)
        const uint64_t kids = __ballot(lane < n && s_par[lane] == cur);  // s_par is shared
        const bool room = len < a.max_path;

        if (a.mode == 0) {
            // ---- greedy: argmax of the target row
            float bv = -__builtin_huge_valf();
            int bi = 0x7fffffff;
            row_pass(prow, V, a.vec, [&](int y, float x) {
                if (x > bv) {  // y increases: a tie keeps the earlier id
                    bv = x;
                    bi = y;
                }
            });
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) {
                const float pv = __shfl_xor(bv, off, 64);
                const int pi = __shfl_xor(bi, off, 64);
                if (pv > bv || (pv == bv && pi < bi)) {
                    bv = pv;
                    bi = pi;
                }
            }
            __syncthreads();
            if (lane == 0) {
                s_bv[wave] = bv;
                s_bi[wave] = bi;
            }
            __syncthreads();
            bv = s_bv[0];
            bi = s_bi[0];
#pragma unroll
            for (int w = 1; w < kAcceptWaves; ++w)
                if (s_bv[w] > bv || (s_bv[w] == bv && s_bi[w] < bi)) {
                    bv = s_bv[w];
                    bi = s_bi[w];
                }
            // the lowest-index child carrying token bi
            uint64_t hit = 0;
            for (uint64_t m = kids; m; m &= m - 1) {
                const int c = __builtin_ctzll(m);
                if (s_tok[c] == bi) {
                    hit = 1ull << c;
                    break;
                }
            }
            if (hit && room) {
                const int c = __builtin_ctzll(hit);
                if (t == 0) a.accepted_idx[(size_t)b * a.max_path + len] = c;
                ++len;
                cur = c;
                continue;
            }
            bonus = bi;
            break;
        }

        // ---- sampling
        const float *qrow = cur < 0 ? a.q_ctx + (size_t)b * V : a.q_node + (size_t)(lo + cur) * V;
        double A = 1.0, C = 0.0, Zp = 1.0, Zq = 1.0;
        int k = 0;  // rejections at this node
        int acc = -1;
        for (uint64_t m = room ? kids : 0ull; m; m &= m - 1) {
            const int c = __builtin_ctzll(m);
            const int x = s_tok[c];
            const double u = (double)a.u_node[lo + c];
            const float px = prow[x], qx = qrow[x];
            const double rpx = residual(px, qx, A, C);
            if (__dmul_rn(__dmul_rn(u, (double)qx), Zp) < __dmul_rn(rpx, Zq)) {
                acc = c;
                break;
            }
            // reject x: new coefficients, then one pass over both rows for the new Zp
            A = A / Zp;
            C = C / Zp + 1.0 / Zq;
            Zq = Zq - (double)qx;
            double part = 0.0;
            for (int y0 = t; y0 < V; y0 += kAcceptThreads * kAcceptBatch) {
                float py[kAcceptBatch], qy[kAcceptBatch];
#pragma unroll
                for (int u2 = 0; u2 < kAcceptBatch; ++u2) {
                    const int y = min(y0 + u2 * kAcceptThreads, V - 1);
                    py[u2] = __builtin_nontemporal_load(prow + y);
                    qy[u2] = __builtin_nontemporal_load(qrow + y);
                }
#pragma unroll
                for (int u2 = 0; u2 < kAcceptBatch; ++u2)
                    if (y0 + u2 * kAcceptThreads < V) part += residual(py[u2], qy[u2], A, C);
            }
            Zp = block_sum_d(part, s_red);
            ++k;
        }
        if (acc >= 0) {
            if (t == 0) a.accepted_idx[(size_t)b * a.max_path + len] = acc;
            ++len;
            cur = acc;
            continue;
        }
        // bonus: smallest y with cumsum(rp)[y] > u * total; thread t owns a contiguous
        // chunk, the chunk sums are scanned in thread order
        const int chunk = (V + kAcceptThreads - 1) / kAcceptThreads;
        const int y0 = min(V, t * chunk), y1 = min(V, y0 + chunk);
        double cs = 0.0;
#pragma unroll 8
        for (int y = y0; y < y1; ++y) cs += k == 0 ? (double)prow[y] : residual(prow[y], qrow[y], A, C);
        s_scan[t] = cs;
        __syncthreads();
        for (int off = 1; off < kAcceptThreads; off <<= 1) {
            const double v = t >= off ? s_scan[t - off] : 0.0;
            __syncthreads();
            s_scan[t] += v;
            __syncthreads();
        }
        const double total = k == 0 ? s_scan[kAcceptThreads - 1] : Zp;
        const double thr = (double)a.u_bonus[b] * total;
        if (t == 0) s_pick = V - 1;
        __syncthreads();
        double run = t > 0 ? s_scan[t - 1] : 0.0;  // exclusive prefix of this chunk
        if (run <= thr) {
            for (int y = y0; y < y1; ++y) {
                run += k == 0 ? (double)prow[y] : residual(prow[y], qrow[y], A, C);
                if (run > thr) {
                    atomicMin(&s_pick, y);
                    break;
                }
            }
        } else if (cs > 0.0) {
            atomicMin(&s_pick, y0);  // the first chunk past the threshold, should rounding
        }                            // hide the crossing from the chunk before it
        __syncthreads();
        bonus = s_pick;
        break;
    }
    if (t == 0) {
        if (a.tree_status) a.tree_status[b] = BOLE_TREE_OK;
        a.accepted_len[b] = len;
        a.bonus[b] = bonus;
    }
    for (int m = len + t; m < a.max_path; m += kAcceptThreads) a.accepted_idx[(size_t)b * a.max_path + m] = -1;
}

hipError_t launch_tree_accept(const float *p_ctx, const float *p_node, const float *q_ctx,
                              const float *q_node, const int32_t *parent, const int32_t *token,
                              const int32_t *node_offsets, const float *u_node,
                              const float *u_bonus, const bole_accept_dims_t &d, int32_t *accepted_idx,
                              int32_t *accepted_len, int32_t *bonus, int32_t *tree_status,
                              hipStream_t stream) {
    AcceptArgs a;
    a.p_ctx = p_ctx;
    a.p_node = p_node;
    a.q_ctx = q_ctx;
    a.q_node = q_node;
    a.u_node = u_node;
    a.u_bonus = u_bonus;
    a.parent = parent;
    a.token = token;
    a.node_offsets = node_offsets;
    a.accepted_idx = accepted_idx;
    a.accepted_len = accepted_len;
    a.bonus = bonus;
    a.tree_status = tree_status;
    a.B = d.batch;
    a.T = d.total_nodes;
    a.V = d.vocab;
    a.max_path = d.max_path;
    a.mode = d.mode;
    a.vec = d.vocab % 4 == 0 &&
            ((reinterpret_cast<uintptr_t>(p_ctx) | reinterpret_cast<uintptr_t>(p_node)) % 16) == 0;
    tree_accept_kernel<<<dim3((unsigned)d.batch), dim3(kAcceptThreads), 0, stream>>>(a);
    return hipGetLastError();
}

}  // namespace bole
