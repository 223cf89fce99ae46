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
//    rejected ones before it: on a rejection of x, p_res <- (p_res - q_res)+ renormalised,
//    and x leaves q_res, renormalised. With rp = p_res * Zp and rq = q_res * Zq
//    unnormalised, x is accepted when u * rq(x) * Zp < rp(x) * Zq. The residuals are
//    never stored: after k rejections rp(y) = max(p(y) A - q(y) C, 0), with A, C, Zq
//    updated per rejection of x as A <- A / Zp, C <- C / Zp + 1 / Zq, Zq <- Zq - q(x), and
//    Zp the sum of the new rp: one pass over the node's two fp32 rows (16-byte loads).
//    This equals the step-by-step residual in real arithmetic because a clamp at 0 never
//    releases and a rejected token's residual is already 0; it needs siblings with
//    distinct tokens (drafts without replacement), so a tree with two siblings carrying
//    one token is reported BOLE_TREE_BAD_TOKEN under sampling. The bonus is drawn from
//    rp by inverse CDF over tiles of 4 elements per thread: per-wavefront tile sums,
//    walked in order until the running sum passes the threshold, then a block-wide prefix
//    sum inside that tile. fp64 throughout, products and differences separately rounded.
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
    bool vec;   // target rows are 16-byte aligned (V % 4 == 0 and aligned bases)
    bool vecq;  // so are the draft rows
};

typedef float f4 __attribute__((ext_vector_type(4)));

// A 16-byte piece of a row: KEEP (sampling, which reads a node's rows again within the
// call) a plain load that leaves the lines in the caches, else a streaming load (greedy
// reads each row once; plain loads there were slower: 75 -> 91 us cold, while sampling
// went 300 -> 251 us).
template <bool KEEP>
__device__ __forceinline__ f4 piece(const float *p) {
    return KEEP ? *reinterpret_cast<const f4 *>(p)
                : __builtin_nontemporal_load(reinterpret_cast<const f4 *>(p));
}

// Elements y .. y+3 of an fp32 row (y a multiple of 4; values past V are unspecified):
// one 16-byte load when the row allows it.
template <bool KEEP>
__device__ __forceinline__ f4 load4(const float *row, int y, int V, bool vec) {
    if (vec) return piece<KEEP>(row + min(y, V - 4));
    f4 x;
#pragma unroll
    for (int c = 0; c < 4; ++c) x[c] = row[min(y + c, V - 1)];
    return x;
}

// Calls f(y, value) for the elements of an fp32 row this thread owns, in increasing y.
// Loads are issued kAcceptBatch at a time before any is used. Positions past the row
// (y >= V) get the value `pad`, which must leave f's result unchanged (-inf for a maximum,
// 0 for a sum): every loaded value is then used unconditionally, so the compiler keeps
// the batch of loads in flight together instead of moving a load under a per-element
// branch.
template <bool KEEP, typename F>
__device__ __forceinline__ void row_pass(const float *row, int V, bool vec, F f, float pad) {
    const int t = threadIdx.x;
    if (vec) {
        constexpr int step = 4 * kAcceptThreads;
        for (int y0 = 4 * t; y0 < V; y0 += step * kAcceptBatch) {
            f4 x[kAcceptBatch];
#pragma unroll
            for (int u = 0; u < kAcceptBatch; ++u) {
                const int y = y0 + u * step;
                x[u] = piece<KEEP>(row + min(y, V - 4));
            }
#pragma unroll
            for (int u = 0; u < kAcceptBatch; ++u) {
                const int y = y0 + u * step;
#pragma unroll
                for (int c = 0; c < 4; ++c) f(y + c, y + c < V ? x[u][c] : pad);
            }
        }
    } else {
        for (int y0 = t; y0 < V; y0 += kAcceptThreads * kAcceptBatch) {
            float x[kAcceptBatch];
#pragma unroll
            for (int u = 0; u < kAcceptBatch; ++u)
                x[u] = row[min(y0 + u * kAcceptThreads, V - 1)];
#pragma unroll
            for (int u = 0; u < kAcceptBatch; ++u) {
                const int y = y0 + u * kAcceptThreads;
                f(y, y < V ? x[u] : pad);
            }
        }
    }
}

// Calls f(y, p(y), q(y)) for the elements of two fp32 rows this thread owns, in
// increasing y; kAcceptBatch / 4 16-byte loads of each row in flight. Positions past the
// rows get p = q = 0 (f must then add nothing), for the reason given above.
template <bool KEEP, typename F>
__device__ __forceinline__ void row_pass2(const float *prow, const float *qrow, int V, bool vec,
                                          F f) {
    constexpr int NB = kAcceptBatch / 4;
    constexpr int step = 4 * kAcceptThreads;
    for (int y0 = 4 * threadIdx.x; y0 < V; y0 += step * NB) {
        f4 px[NB], qx[NB];
#pragma unroll
        for (int u = 0; u < NB; ++u) {
            px[u] = load4<KEEP>(prow, y0 + u * step, V, vec);
            qx[u] = load4<KEEP>(qrow, y0 + u * step, V, vec);
        }
#pragma unroll
        for (int u = 0; u < NB; ++u) {
            const int y = y0 + u * step;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const bool in = y + c < V;
                f(y + c, in ? px[u][c] : 0.f, in ? qx[u][c] : 0.f);
            }
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

__device__ __forceinline__ double wave_sum_d(double x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
    return x;
}

// Inclusive prefix sum over the wavefront's lanes, in lane order.
__device__ __forceinline__ double wave_scan_d(double x) {
    const int lane = lane_id();
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const double y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
    }
    return x;
}

// The bonus search works on tiles of kTile elements, 4 per thread; tile sums are formed
// per wavefront and kept for kTileGroup tiles at a time.
constexpr int kTile = 4 * kAcceptThreads;
constexpr int kTileGroup = 32;
constexpr int kTileBatch = kAcceptBatch / 4;

// VP, VQ: the target rows (p), the draft rows (q) take 16-byte loads. As template
// constants they leave no branch between the loads of a batch.
template <bool VP, bool VQ, bool KEEP>
__global__ __launch_bounds__(kAcceptThreads) void tree_accept_kernel(AcceptArgs a) {
    __shared__ double s_red[kAcceptWaves];
    __shared__ double s_tw[kAcceptWaves][kTileGroup];
    __shared__ double s_before;
    __shared__ int s_tile;
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
        if (st == BOLE_TREE_OK && a.mode == BOLE_ACCEPT_SAMPLE) {
            // sampling tests siblings as drafts without replacement: two siblings with
            // one token make a malformed tree
            bool dup = false;
            for (int j = 0; j < n; ++j) {  // n is wave-uniform
                const int pj = __shfl(p, j, 64), tj = __shfl(tk, j, 64);
                dup |= j < lane && lane < n && pj == p && tj == tk;
            }
            if (__any(dup)) st = BOLE_TREE_BAD_TOKEN;
        }
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
            row_pass<KEEP>(prow, V, VP, [&](int y, float x) {
                if (x > bv) {  // y increases: a tie keeps the earlier id
                    bv = x;
                    bi = y;
                }
            }, -__builtin_huge_valf());
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
            row_pass2<KEEP>(prow, qrow, V, VP && VQ,
                      [&](int, float py, float qy) { part += residual(py, qy, A, C); });
            Zp = block_sum_d(part, s_red);
            ++k;
        }
        if (acc >= 0) {
            if (t == 0) a.accepted_idx[(size_t)b * a.max_path + len] = acc;
            ++len;
            cur = acc;
            continue;
        }
        // bonus: smallest y with cumsum(rp)[y] > u * total (total = sum(p) at a fresh
        // node, else Zp). Tiles of kTile elements in order: per-wavefront tile sums, and
        // thread 0 walks the tile sums until the running sum passes the threshold; inside
        // that tile, a block-wide prefix sum in thread order finds the element.
        const bool withq = k > 0;
        auto rval = [&](float p, float q) -> double { return withq ? residual(p, q, A, C) : (double)p; };
        double total = Zp;
        if (!withq) {
            double part = 0.0;
            row_pass<KEEP>(prow, V, VP, [&](int, float x) { part += (double)x; }, 0.f);
            total = block_sum_d(part, s_red);
        }
        const double thr = (double)a.u_bonus[b] * total;
        const int ntiles = (V + kTile - 1) / kTile;
        if (t == 0) {
            s_before = 0.0;
            s_tile = -1;
            s_pick = V - 1;  // the last y if rounding leaves no crossing
        }
        int tile = -1;
        for (int g0 = 0; g0 < ntiles; g0 += kTileGroup) {
            const int gn = min(kTileGroup, ntiles - g0);
            for (int j0 = 0; j0 < gn; j0 += kTileBatch) {
                f4 pv[kTileBatch], qv[kTileBatch];
#pragma unroll
                for (int u = 0; u < kTileBatch; ++u) {
                    const int y = (g0 + j0 + u) * kTile + 4 * t;
                    pv[u] = load4<KEEP>(prow, y, V, VP);
                    qv[u] = withq ? load4<KEEP>(qrow, y, V, VQ) : f4{0.f, 0.f, 0.f, 0.f};
                }
#pragma unroll
                for (int u = 0; u < kTileBatch; ++u) {
                    if (j0 + u >= gn) break;  // uniform
                    const int y = (g0 + j0 + u) * kTile + 4 * t;
                    double sv = 0.0;
#pragma unroll
                    for (int c = 0; c < 4; ++c)  // past the row: + 0, exact
                        sv += y + c < V ? rval(pv[u][c], qv[u][c]) : 0.0;
                    sv = wave_sum_d(sv);
                    if (lane == 0) s_tw[wave][j0 + u] = sv;
                }
            }
            __syncthreads();
            if (t == 0) {
                double run = s_before;
                for (int jj = 0; jj < gn; ++jj) {
                    double S = 0.0;
                    for (int w = 0; w < kAcceptWaves; ++w) S += s_tw[w][jj];
                    if (run + S > thr) {
                        s_tile = g0 + jj;
                        break;
                    }
                    run += S;
                }
                s_before = run;  // the sum over the tiles before the crossing one
            }
            __syncthreads();
            tile = s_tile;
            if (tile >= 0) break;  // uniform
        }
        if (tile >= 0) {
            const int y = tile * kTile + 4 * t;
            const f4 pv = load4<KEEP>(prow, y, V, VP);
            const f4 qv = withq ? load4<KEEP>(qrow, y, V, VQ) : f4{0.f, 0.f, 0.f, 0.f};
            double e[4], sv = 0.0;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                e[c] = y + c < V ? rval(pv[c], qv[c]) : 0.0;
                sv += e[c];
            }
            const double incl = wave_scan_d(sv);
            double wex = __shfl_up(incl, 1, 64);
            if (lane == 0) wex = 0.0;
            if (lane == 63) s_red[wave] = incl;
            __syncthreads();
            double run = s_before;
            for (int w = 0; w < wave; ++w) run += s_red[w];
            run += wex;  // the sum over every element before this thread's first
            if (run <= thr) {
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    run += e[c];
                    if (run > thr) {
                        atomicMin(&s_pick, y + c);
                        break;
                    }
                }
            } else {
                // the crossing fell before this thread, hidden by rounding from the one
                // holding it: its first positive element
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    if (e[c] > 0.0) {
                        atomicMin(&s_pick, y + c);
                        break;
                    }
            }
        }
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
    a.vecq = d.vocab % 4 == 0 && q_ctx && q_node &&
             ((reinterpret_cast<uintptr_t>(q_ctx) | reinterpret_cast<uintptr_t>(q_node)) % 16) == 0;
    const dim3 grid((unsigned)d.batch), block(kAcceptThreads);
    if (a.mode == BOLE_ACCEPT_SAMPLE) {
        if (a.vec && a.vecq) tree_accept_kernel<true, true, true><<<grid, block, 0, stream>>>(a);
        else if (a.vec) tree_accept_kernel<true, false, true><<<grid, block, 0, stream>>>(a);
        else if (a.vecq) tree_accept_kernel<false, true, true><<<grid, block, 0, stream>>>(a);
        else tree_accept_kernel<false, false, true><<<grid, block, 0, stream>>>(a);
    } else {
        // greedy reads no draft rows
        if (a.vec) tree_accept_kernel<true, false, false><<<grid, block, 0, stream>>>(a);
        else tree_accept_kernel<false, false, false><<<grid, block, 0, stream>>>(a);
    }
    return hipGetLastError();
}

}  // namespace bole
