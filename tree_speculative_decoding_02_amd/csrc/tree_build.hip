// tree_build.hip - draft-tree construction from a block drafter's position-wise
// marginals and the online budget controller (BASTION summary page: section 1 path
// score, section 2 best-first expansion, section 3 budget controller).
//
// Three launches:
//  1. topk_slice_kernel: the top 64 entries of every (sequence, position) row, per
//     vocabulary slice, ordered by (probability desc, index asc). The only HBM-heavy
//     step: it streams the marginals once.
//  2. build_kernel: one wavefront per sequence merges its slices' lists per position,
//     grows the best-first tree (lane = candidate source) and runs the controller.
//  3. pack_kernel: one workgroup scans the kept sizes into node_offsets and packs the
//     trees.
// Only the top 64 tokens of a position can ever be used: one parent's children are
// inserted in rank order and a tree has at most 64 nodes.
#include <algorithm>
#include <mutex>

#include "bole_device.h"
#include "launch.h"

namespace bole {

constexpr int kTopK = 64;
constexpr int kBuildThreads = 256;
constexpr int kMaxDepth = 32;
constexpr int kMaxBudget = 64;

// Orderable key of a probability (finite, >= 0): its bits without the sign, plus one. A
// larger value has a larger key, -0 ranks as +0, and key 0 marks "no element".
__device__ __forceinline__ uint32_t bits2key(uint32_t u) { return (u & 0x7fffffffu) + 1u; }
__device__ __forceinline__ float key2f(uint32_t k) { return __uint_as_float(k - 1u); }
// rank order: larger key first, then lower index (indices are >= 0): one 64-bit compare
// of (key, ~index), with no branches
__device__ __forceinline__ bool better(uint32_t ka, int ia, uint32_t kb, int ib) {
    return (((uint64_t)ka << 32) | (uint32_t)~ia) > (((uint64_t)kb << 32) | (uint32_t)~ib);
}

// One compare-exchange step of a 64-lane bitonic network: the lower lane of each pair
// keeps the better element when `desc`, the worse otherwise.
__device__ __forceinline__ void bitonic_step(uint32_t &k, int &i, int j, bool desc) {
    const int lane = lane_id();
    const uint32_t pk = __shfl_xor(k, j, 64);
    const int pi = __shfl_xor(i, j, 64);
    const bool keep_better = ((lane & j) == 0) == desc;
    const bool pb = better(pk, pi, k, i);
    if (keep_better ? pb : !pb) {
        k = pk;
        i = pi;
    }
}

// Sorts the 64 lane values in rank order (lane 0 the best).
__device__ __forceinline__ void wave_sort64(uint32_t &k, int &i) {
    const int lane = lane_id();
#pragma unroll
    for (int size = 2; size <= 64; size <<= 1)
#pragma unroll
        for (int j = size >> 1; j > 0; j >>= 1) bitonic_step(k, i, j, (lane & size) == 0);
}

// (k, i) sorted in rank order across lanes; merges another sorted list (nk, ni) and
// keeps the best 64, sorted.
__device__ __forceinline__ void wave_merge64(uint32_t &k, int &i, uint32_t nk, int ni) {
    const int lane = lane_id();
    const uint32_t rk = __shfl(nk, 63 - lane, 64);
    const int ri = __shfl(ni, 63 - lane, 64);
    if (better(rk, ri, k, i)) {
        k = rk;
        i = ri;
    }
#pragma unroll
    for (int j = 32; j > 0; j >>= 1) bitonic_step(k, i, j, true);
}

// ---- 1. top 64 of one vocabulary slice of one (sequence, position) row
//
// The workgroup streams its slice [lo, hi) in chunks of kChunk elements, the next chunk's
// loads in flight while the current one is filtered, and each wavefront keeps candidates
// of its own: wavefront w holds, of the chunk at c0, the elements c0 + kSub w + (64 j + l) W
// + c of lane l (j < kChunkPerThread / W, c < W) as orderable keys, and gathers those at or
// above a running threshold theta into its own LDS buffer (slots from a ballot; the count
// is the same in every lane, so no atomics).
//  - theta starts as the smallest, over the wavefronts, of each wavefront's 16th largest
//    lane maximum in the first chunk (a 32-step ballot search; at least 64 elements reach
//    it), the one barrier before the end.
//  - A wavefront whose buffer passes half full raises theta to its 64th largest buffered
//    key resolved to its top kThetaBits bits (a bitwise search), drops the candidates below
//    it and publishes it in LDS; every wavefront takes the largest published value before
//    each chunk. Each such value is at most the 64th largest key seen in the slice, so the
//    slice's top 64 always stay in the buffers; a value read while it is being raised is
//    an earlier, smaller one, which is as safe, so these exchanges need no barrier.
//  - At the end each wavefront ranks its candidates and writes its best 64 to LDS, and
//    wavefront 0 merges the four lists.
// A wavefront whose buffer overflows (many keys equal to theta, such as uniform rows) takes
// 64 rounds of extraction over its own elements, read again. (A first version shared one
// buffer per workgroup, with a barrier per chunk and one per bit of each threshold search:
// 57.8 us for the benchmark's 512 rows x 128,256.)
constexpr int kChunkPerThread = 16;
constexpr int kThetaBits = 16;  // key bits resolved by a threshold search
constexpr int kChunk = kBuildThreads * kChunkPerThread;  // 4096 elements
constexpr int kSub = 64 * kChunkPerThread;              // 1024: a wavefront's part of a chunk
constexpr int kWaveCap = 512;                           // candidates per wavefront

// The 64th largest of the wavefront's J x W values per lane, resolved to its top
// kThetaBits bits and never above it (0 when fewer than 64 values are nonzero).
template <int J, int W, typename VT>
__device__ __forceinline__ uint32_t wave_theta64(const VT (&v)[J]) {
    uint32_t th = 0u;
    for (int bit = 31; bit >= 32 - kThetaBits; --bit) {
        const uint32_t cand = th | (1u << bit);
        int c = 0;
#pragma unroll
        for (int j = 0; j < J; ++j)
#pragma unroll
            for (int e = 0; e < W; ++e) c += __popcll(__ballot(v[j][e] >= cand));
        if (c >= kTopK) th = cand;
    }
    return th;
}

template <int W>
__global__ __launch_bounds__(kBuildThreads) void topk_slice_kernel(
    const float *__restrict__ marginals, uint2 *__restrict__ lists, int V, int S, int slice_len) {
    constexpr int J = kChunkPerThread / W;
    constexpr int R = kWaveCap / 64;  // buffer entries per lane
    typedef uint32_t uv __attribute__((ext_vector_type(W)));
    __shared__ uint32_t s_k[4][kWaveCap];
    __shared__ int s_i[4][kWaveCap];
    __shared__ uint32_t s_lk[4][kTopK];  // each wavefront's best 64, in rank order
    __shared__ int s_li[4][kTopK];
    __shared__ uint32_t s_th4[4];        // first chunk: each wavefront's 16th largest lane maximum
    __shared__ uint32_t s_theta[4];      // each wavefront's published threshold
    const int t = threadIdx.x, lane = lane_id(), wave = t >> 6;
    const size_t row = blockIdx.x / S;
    const int slice = blockIdx.x - (int)row * S;
    const int lo = slice * slice_len, hi = min(V, lo + slice_len);
    const float *src = marginals + row * (size_t)V;
    uint2 *dst = lists + (size_t)blockIdx.x * kTopK;
    uint32_t *const bk_s = s_k[wave];
    int *const bi_s = s_i[wave];

    // first element of load j of this lane, in this wavefront's part of the chunk at c0
    auto elem = [&](int c0, int j) { return c0 + kSub * wave + (j * 64 + lane) * W; };
    // a chunk's raw bits (addresses clamped into the row)
    auto load = [&](int c0, uv (&x)[J]) {
#pragma unroll
        for (int j = 0; j < J; ++j)
            x[j] = __builtin_nontemporal_load(
                reinterpret_cast<const uv *>(src + (uint32_t)min(elem(c0, j), V - W)));
    };
    // the keys in place (0 outside the slice: only the last chunk masks), and the lane's
    // largest
    auto keys = [&](int c0, uv (&x)[J]) -> uint32_t {
        uint32_t mx = 0u;
        const bool whole = c0 + kChunk <= hi;
#pragma unroll
        for (int j = 0; j < J; ++j)
#pragma unroll
            for (int c = 0; c < W; ++c) {
                x[j][c] = (whole || elem(c0, j) + c < hi) ? bits2key(x[j][c]) : 0u;
                mx = max(mx, x[j][c]);
            }
        return mx;
    };

    int cnt = 0;  // candidates in this wavefront's buffer (the same in every lane)
    uint32_t theta = 1u;
    // gathers the keys >= theta of one chunk part; the count goes on past the capacity
    // (the entries past it are not written), which marks an overflow
    auto gather = [&](int c0, uv (&x)[J], uint32_t mx) {
        if (!__ballot(mx >= theta)) return;
#pragma unroll
        for (int j = 0; j < J; ++j) {
            int sbase = elem(c0, j);
            asm volatile("" : "+v"(sbase));  // recomputed per load, not held in registers
#pragma unroll
            for (int c = 0; c < W; ++c) {
                const bool take = x[j][c] >= theta;
                const uint64_t m = __ballot(take);
                if (m) {
                    const int slot = cnt + (int)__builtin_amdgcn_mbcnt_hi(
                                               (uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
                    if (take && slot < kWaveCap) {
                        bk_s[slot] = x[j][c];
                        bi_s[slot] = sbase + c;
                    }
                    cnt += (int)__popcll(m);
                }
            }
        }
    };
    // theta <- max(theta, the 64th largest buffered key resolved to kThetaBits bits); the
    // candidates below it are dropped (read into registers first, so in place)
    // (the kept entries move only toward the front: entry r of each lane is read before any
    // write reaches its slot)
    auto compact = [&]() {
        uint32_t bk[R][1];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int x2 = lane + 64 * r;
            bk[r][0] = x2 < cnt ? bk_s[x2] : 0u;
        }
        theta = max(theta, wave_theta64<R, 1>(bk));
        if (lane == 0) s_theta[wave] = theta;
        int nc = 0;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int x2 = lane + 64 * r;
            const bool keep = bk[r][0] >= theta;
            const int ix = keep ? bi_s[x2] : 0;
            const uint64_t m = __ballot(keep);
            const int slot = nc + (int)__builtin_amdgcn_mbcnt_hi(
                                      (uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
            if (keep) {
                bk_s[slot] = bk[r][0];
                bi_s[slot] = ix;
            }
            nc += (int)__popcll(m);
        }
        cnt = nc;
    };
    // one chunk part: false when the buffer overflowed
    auto step = [&](int c0, uv (&x)[J], uint32_t mx) -> bool {
        theta = max(max(theta, max(s_theta[0], s_theta[1])), max(s_theta[2], s_theta[3]));
        gather(c0, x, mx);
        if (cnt > kWaveCap) return false;
        if (cnt > kWaveCap / 2) compact();
        return true;
    };

    uv A[J], B2[J];  // two chunk buffers, alternating
    load(lo, A);
    if (lo + kChunk < hi) load(lo + kChunk, B2);
    uint32_t mx0 = keys(lo, A);
    {
        // the wavefront's 16th largest lane maximum in the first chunk, bit by bit
        uint32_t th = 0u;
        for (int bit = 31; bit >= 0; --bit) {
            const uint32_t cand = th | (1u << bit);
            if (__popcll(__ballot(mx0 >= cand)) >= 16) th = cand;
        }
        if (lane == 0) {
            s_th4[wave] = th;
            s_theta[wave] = 1u;
        }
    }
    __syncthreads();
    // >= 1: a key at or above it is never the empty key
    theta = max(1u, min(min(s_th4[0], s_th4[1]), min(s_th4[2], s_th4[3])));
    bool overflow = false;
    for (int c0 = lo; c0 < hi; c0 += 2 * kChunk) {
        // chunk c0 in A (keys formed), chunk c0 + kChunk in flight in B2
        if (!step(c0, A, mx0)) {
            overflow = true;
            break;
        }
        const int c1 = c0 + kChunk;
        if (c1 >= hi) break;
        if (c1 + kChunk < hi) load(c1 + kChunk, A);
        const uint32_t mx1 = keys(c1, B2);
        if (!step(c1, B2, mx1)) {
            overflow = true;
            break;
        }
        if (c1 + kChunk >= hi) break;
        if (c1 + 2 * kChunk < hi) load(c1 + 2 * kChunk, B2);
        mx0 = keys(c1 + kChunk, A);
    }

    if (!overflow) {
        if (cnt > 2 * kTopK) compact();  // a short ranking
        // each candidate's rank is the number of better ones ((key, index) pairs are
        // distinct, so ranks are too)
        for (int x = lane; x < cnt; x += 64) {
            const uint32_t kx = bk_s[x];
            const int ix = bi_s[x];
            int rank = 0;
            for (int y = 0; y < cnt; ++y) rank += better(bk_s[y], bi_s[y], kx, ix) ? 1 : 0;
            if (rank < kTopK) {
                s_lk[wave][rank] = kx;
                s_li[wave][rank] = ix;
            }
        }
        for (int r = cnt + lane; r < kTopK; r += 64) {
            s_lk[wave][r] = 0u;
            s_li[wave][r] = 0x7fffffff;
        }
    } else {
        // many ties: 64 rounds, each taking the best of this wavefront's elements not yet
        // taken (ranking after the last one taken), read again
        uint32_t lk = 0xffffffffu;
        int li = -1;
        for (int r = 0; r < kTopK; ++r) {
            uint32_t bk2 = 0u;
            int bi = 0x7fffffff;
            for (int c0 = lo; c0 < hi; c0 += kChunk)
                for (int j = 0; j < J; ++j)
                    for (int c = 0; c < W; ++c) {
                        const int e = elem(c0, j) + c;
                        if (e < hi) {
                            const uint32_t k = bits2key(__float_as_uint(src[e]));
                            if (better(lk, li, k, e) && better(k, e, bk2, bi)) {
                                bk2 = k;
                                bi = e;
                            }
                        }
                    }
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) {
                const uint32_t pk = __shfl_xor(bk2, off, 64);
                const int pi = __shfl_xor(bi, off, 64);
                if (better(pk, pi, bk2, bi)) {
                    bk2 = pk;
                    bi = pi;
                }
            }
            if (lane == 0) {
                s_lk[wave][r] = bk2;
                s_li[wave][r] = bk2 ? bi : 0x7fffffff;
            }
            lk = bk2;
            li = bi;
        }
    }
    __syncthreads();
    if (wave == 0) {
        uint32_t k = s_lk[0][lane];
        int i = s_li[0][lane];
#pragma unroll
        for (int w = 1; w < 4; ++w) wave_merge64(k, i, s_lk[w][lane], s_li[w][lane]);
        dst[lane] = make_uint2(k, (uint32_t)i);
    }
}

// Best offer over the wavefront. An offer's key is the score's bits + 1 (scores are
// >= +0, so this orders them; 0 means no offer). The largest key comes from a DPP maximum
// toward lane 63 (row_shr 1, 2, 4, 8 within each row of 16, then row_bcast 15 and 31
// across rows; lanes whose DPP source is outside the row or masked contribute 0); equal
// scores go to the earlier source, the context (source -1, lane 63) first, by a ballot.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ void max_dpp_step(uint32_t &x) {
    const uint32_t p = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, ROW_MASK, 0xf, false);
    x = max(x, p);
}

// The best key (wave-uniform) and its source's lane: lane 63 when the context offers
// it, else the lowest lane that does.
__device__ __forceinline__ uint32_t wave_bestkey(uint32_t key, int &best_lane) {
    uint32_t x = key;
    max_dpp_step<0x111, 0xf>(x);  // row_shr:1
    max_dpp_step<0x112, 0xf>(x);  // row_shr:2
    max_dpp_step<0x114, 0xf>(x);  // row_shr:4
    max_dpp_step<0x118, 0xf>(x);  // row_shr:8
    max_dpp_step<0x142, 0xa>(x);  // row_bcast:15 into rows 1 and 3
    max_dpp_step<0x143, 0xc>(x);  // row_bcast:31 into rows 2 and 3
    const uint32_t best = (uint32_t)__builtin_amdgcn_readlane((int)x, 63);
    const uint64_t at = __ballot(key == best);
    best_lane = (at >> 63) ? 63 : __builtin_ctzll(at);
    return best;
}

// ---- 2. best-first tree and controller, one wavefront per sequence
//
// Lane l < n is tree node l as a candidate source (its depth, next child rank, score);
// lane 63 is the verified context, whose children are the depth-1 tokens. Each step every
// source offers its best child not yet inserted, score fp32(rho_source * q); the best
// offer (score desc, source asc with the context as -1) becomes node n. Node n's outputs
// are kept in lane n's output registers (which do not alias the context's state in
// lane 63).
__global__ __launch_bounds__(256) void build_kernel(
    const uint2 *__restrict__ lists, const float *__restrict__ cost, float l_ar, int D, int S,
    int n_max, int fixed, int32_t *__restrict__ n_nodes, int32_t *__restrict__ par_out,
    int32_t *__restrict__ tok_out, float *__restrict__ rho_out, float *__restrict__ speedup) {
    __shared__ float s_val[kMaxDepth][kTopK];
    __shared__ int s_tok[kMaxDepth][kTopK];
    const int lane = lane_id(), wave = threadIdx.x >> 6;
    const int b = blockIdx.x;

    // per-position candidate lists: wavefront w merges positions w, w + 4, ..., loading
    // up to 8 slice lists at a time
    constexpr int kBatch = 8;
    for (int d = wave; d < D; d += 4) {
        const uint2 *l0 = lists + ((size_t)b * D + d) * S * kTopK;
        uint32_t k = 0u;
        int i = 0x7fffffff;
        for (int s0 = 0; s0 < S; s0 += kBatch) {
            uint2 x[kBatch];
#pragma unroll
            for (int u = 0; u < kBatch; ++u)
                x[u] = s0 + u < S ? l0[(size_t)(s0 + u) * kTopK + lane] : make_uint2(0u, 0x7fffffffu);
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
                if (s0 + u == 0) {
                    k = x[u].x;
                    i = (int)x[u].y;
                } else if (s0 + u < S) {
                    wave_merge64(k, i, x[u].x, (int)x[u].y);
                }
            }
        }
        s_val[d][lane] = k ? key2f(k) : -1.f;  // -1: no candidate of this rank
        s_tok[d][lane] = i;
    }
    __syncthreads();
    if (wave != 0) return;
    // C(N) for N = lane + 1
    const float c_lane = (cost != nullptr && lane < n_max) ? cost[lane] : 1.f;

    // source state (lane 63: the context): depth, rank and score of its next child, the
    // value of that child (cur) and of the one after it (nxt), so that no LDS read sits
    // on a step's critical path: only a winning lane refills nxt, and it is needed only
    // when that lane wins again. A new node's first two candidates come from the
    // per-position registers f0, f1 (lane d: the two best of position d + 1).
    const float f0 = lane < D ? s_val[lane][0] : -1.f;
    const float f1 = lane < D ? s_val[lane][1] : -1.f;
    int src_depth = 0, src_rank = 0;
    float src_rho = 1.f;
    float cur = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(f0), 0));
    float nxt = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(f1), 0));
    int o_par = -1, o_d = 0, o_r = 0;  // node outputs: parent, the candidate's position and rank
    float o_rho = 0.f;
    int n = 0;
    for (; n < n_max; ++n) {
        const bool is_src = lane < n || lane == 63;
        const bool offer = is_src && cur >= 0.f;
        const float sc = __fmul_rn(src_rho, cur);
        const uint32_t key = offer ? __float_as_uint(sc) + 1u : 0u;
        int wl;  // the winning source's lane
        const uint32_t best = wave_bestkey(key, wl);
        if (best == 0u) break;  // no source offers a child (wave-uniform)
        const float bs = __uint_as_float(best - 1u);
        const int bw = wl == 63 ? -1 : wl;  // the winning source: -1 for the context
        const int wd = __builtin_amdgcn_readlane(src_depth, wl);
        const int wr = __builtin_amdgcn_readlane(src_rank, wl);
        if (lane == wl) {
            ++src_rank;
            cur = nxt;
            nxt = src_rank + 1 < kTopK ? s_val[src_depth][src_rank + 1] : -1.f;
        }
        const int dn = wd + 1;  // the new node's depth; its children are at position dn + 1
        const float g0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(f0), dn < D ? dn : 0));
        const float g1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(f1), dn < D ? dn : 0));
        if (lane == n) {
            o_par = bw < 0 ? -1 : bw;
            o_d = wd;
            o_r = wr;
            o_rho = bs;
            if (n < 63) {
                src_depth = dn;
                src_rank = 0;
                src_rho = bs;
                cur = dn < D ? g0 : -1.f;
                nxt = dn < D ? g1 : -1.f;
            }
        }
    }
    const int built = n;

    // controller: A_hat summed in insertion order, S(N) = A_hat(N) * L_AR / C(N). The sum
    // runs serially (its order fixes the rounding); lane N - 1 keeps A_hat(N), and every
    // S(N) is then formed at once. The tree keeps N - 1 nodes at the first N > 1 with
    // S(N) < S(N - 1) (all of them under a fixed budget).
    int keep = built;
    float s_keep = 0.f;
    if (built > 0 && cost != nullptr) {
        float A = 0.f, a_lane = 0.f;
        for (int N = 1; N <= built; ++N) {
            A = __fadd_rn(A, __int_as_float(__builtin_amdgcn_readlane(__float_as_int(o_rho), N - 1)));
            if (lane == N - 1) a_lane = A;
        }
        const float s_lane = __fdiv_rn(__fmul_rn(a_lane, l_ar), c_lane);  // S(lane + 1)
        const float s_before = __shfl_up(s_lane, 1, 64);                   // S(lane)
        const uint64_t drop = __ballot(!fixed && lane >= 1 && lane < built && s_lane < s_before);
        if (drop) keep = __builtin_ctzll(drop);  // S(keep + 1) < S(keep): keep nodes 0 .. keep - 1
        s_keep = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(s_lane), keep - 1));  // S at the kept size
    }
    if (lane < keep) {
        par_out[(size_t)b * n_max + lane] = o_par;
        tok_out[(size_t)b * n_max + lane] = s_tok[o_d][o_r];
        rho_out[(size_t)b * n_max + lane] = o_rho;
    }
    if (lane == 0) {
        n_nodes[b] = keep;
        if (speedup) speedup[b] = s_keep;
    }
}

// ---- 3. node_offsets and packed trees, one workgroup. The first slots' inputs do not
// depend on the offsets, so their loads are issued before the scan; the scan is one
// shuffle scan per wavefront plus one barrier; the offsets and counts of up to
// kPackLdsSeqs sequences are kept in LDS for the scatter (beyond that, read back from
// node_offsets, which this workgroup wrote before its barrier).
constexpr int kPackThreads = 1024;
constexpr int kPackPre = 4;          // slots per thread loaded ahead of the scan
constexpr int kPackLdsSeqs = 4096;

__global__ __launch_bounds__(kPackThreads) void pack_kernel(
    const int32_t *__restrict__ n_nodes, const int32_t *__restrict__ par_in,
    const int32_t *__restrict__ tok_in, const float *__restrict__ rho_in, int B, int n_max,
    int32_t *__restrict__ node_offsets, int32_t *__restrict__ parent, int32_t *__restrict__ token,
    float *__restrict__ rho) {
    __shared__ int s_wave[kPackThreads / 64];
    __shared__ int s_off[kPackLdsSeqs], s_cnt[kPackLdsSeqs];
    const int t = threadIdx.x, lane = lane_id(), wave = t >> 6;
    const int total = B * n_max;
    int pp[kPackPre], pt[kPackPre];
    float pr[kPackPre];
#pragma unroll
    for (int u = 0; u < kPackPre; ++u) {
        const int x = t + kPackThreads * u;
        pp[u] = 0;
        pt[u] = 0;
        pr[u] = 0.f;
        if (x < total) {
            pp[u] = par_in[x];
            pt[u] = tok_in[x];
            if (rho) pr[u] = rho_in[x];
        }
    }
    const int per = (B + kPackThreads - 1) / kPackThreads;
    const int b0 = min(B, t * per), b1 = min(B, b0 + per);
    int sum = 0;
    for (int b = b0; b < b1; ++b) sum += n_nodes[b];
    // inclusive scan of the per-thread sums within the wavefront, then over wavefronts
    int incl = sum;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(incl, o, 64);
        if (lane >= o) incl += y;
    }
    if (lane == 63) s_wave[wave] = incl;
    __syncthreads();
    int base = 0;
    for (int w = 0; w < wave; ++w) base += s_wave[w];
    int off = base + incl - sum;
    for (int b = b0; b < b1; ++b) {
        const int c = n_nodes[b];
        node_offsets[b] = off;
        if (b < kPackLdsSeqs) {
            s_off[b] = off;
            s_cnt[b] = c;
        }
        off += c;
    }
    if (t == kPackThreads - 1) node_offsets[B] = base + incl;
    __syncthreads();  // offsets and counts (LDS, and node_offsets) visible to the workgroup
    // every (sequence, node) slot in parallel
    auto put = [&](int x, int pv, int tv, float rv) {
        const int b = x / n_max, j = x - b * n_max;
        const int c = b < kPackLdsSeqs ? s_cnt[b] : n_nodes[b];
        if (j < c) {
            const int o = (b < kPackLdsSeqs ? s_off[b] : node_offsets[b]) + j;
            parent[o] = pv;
            token[o] = tv;
            if (rho) rho[o] = rv;
        }
    };
#pragma unroll
    for (int u = 0; u < kPackPre; ++u) {
        const int x = t + kPackThreads * u;
        if (x < total) put(x, pp[u], pt[u], pr[u]);
    }
    for (int x = t + kPackThreads * kPackPre; x < total; x += kPackThreads)
        put(x, par_in[x], tok_in[x], rho ? rho_in[x] : 0.f);
}

// ---- host side
struct BuildLayout {
    size_t lists, n_nodes, par, tok, rho, total;
    int S, slice_len;
};

// Slices per row: about 1024 workgroups in all, each slice at least 8192 elements and a
// multiple of the chunk. At 64 x 8 rows of 128,256 tokens that is two slices per row, four
// workgroups per CU, all resident at once: the whole call took 74.3-74.9 us against 80.0
// with four slices per row (part of that grid ran as a second, partial round), 80.9-81.4
// with one, and 82-91 with three, five or eight.
static void slices_for(const bole_build_dims_t &d, int &S, int &slice_len) {
    const int64_t rows = (int64_t)d.batch * d.depth;
    const int64_t by_grid = rows > 0 ? (1024 + rows - 1) / rows : 1;
    const int64_t by_size = ((int64_t)d.vocab + 8191) / 8192;
    const int64_t want = std::max<int64_t>(1, std::min(by_grid, by_size));
    int64_t len = ((int64_t)d.vocab + want - 1) / want;
    len = (len + kChunk - 1) / kChunk * kChunk;
    slice_len = (int)len;
    S = (int)(((int64_t)d.vocab + len - 1) / len);
}

static BuildLayout build_layout(const bole_build_dims_t &d) {
    BuildLayout L;
    slices_for(d, L.S, L.slice_len);
    auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
    const size_t B = (size_t)d.batch;
    L.lists = 0;
    L.n_nodes = al(B * d.depth * L.S * kTopK * sizeof(uint2));
    L.par = L.n_nodes + al(B * sizeof(int32_t));
    L.tok = L.par + al(B * d.n_max * sizeof(int32_t));
    L.rho = L.tok + al(B * d.n_max * sizeof(int32_t));
    L.total = L.rho + al(B * d.n_max * sizeof(float));
    return L;
}

bool build_dims_ok(const bole_build_dims_t &d) {
    if (d.batch < 0 || d.depth < 1 || d.depth > kMaxDepth || d.vocab < 1 || d.n_max < 1 ||
        d.n_max > kMaxBudget || (d.flags & ~BOLE_BUILD_FIXED_BUDGET))
        return false;
    int S, len;
    slices_for(d, S, len);
    return (uint64_t)d.batch * d.depth * S < (1ull << 31);
}

size_t build_workspace_bytes(const bole_build_dims_t &d) { return build_layout(d).total; }

// Scratch of bole_build_tree_noalloc: the workspace of the three launches, held by the
// library instead of the caller. Every GPU the library runs on has its own copy until the
// process ends. The kernels write every byte they later read (slice lists padded to 64
// entries, per-sequence counts, the kept nodes), so nothing is cleared between calls; two
// calls that overlap on one GPU share the array and race.
static __device__ __align__(256) char scratch[kBuildScratchBytes];

constexpr int kMaxScratchDevices = 64;

hipError_t build_scratch(void **out) {
    static std::mutex mu;
    static void *ptrs[kMaxScratchDevices] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (ptrs[dev] == nullptr) {
        // the name `scratch` stands for a host-side handle: the device address is looked
        // up once per GPU, with that GPU current, and used for every launch after
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        ptrs[dev] = p;
    }
    *out = ptrs[dev];
    return hipSuccess;
}

hipError_t launch_build_tree(const float *marginals, const float *cost, float l_ar,
                             void *workspace, const bole_build_dims_t &d, int32_t *node_offsets,
                             int32_t *parent, int32_t *token, float *rho, float *speedup,
                             hipStream_t stream) {
    const BuildLayout L = build_layout(d);
    char *ws = static_cast<char *>(workspace);
    uint2 *lists = reinterpret_cast<uint2 *>(ws + L.lists);
    int32_t *nn = reinterpret_cast<int32_t *>(ws + L.n_nodes);
    int32_t *par = reinterpret_cast<int32_t *>(ws + L.par);
    int32_t *tok = reinterpret_cast<int32_t *>(ws + L.tok);
    float *rh = reinterpret_cast<float *>(ws + L.rho);
    const unsigned rows = (unsigned)d.batch * (unsigned)d.depth * (unsigned)L.S;
    const bool vec = d.vocab % 4 == 0 && reinterpret_cast<uintptr_t>(marginals) % 16 == 0;
    if (vec)
        topk_slice_kernel<4><<<dim3(rows), dim3(kBuildThreads), 0, stream>>>(marginals, lists, d.vocab, L.S, L.slice_len);
    else
        topk_slice_kernel<1><<<dim3(rows), dim3(kBuildThreads), 0, stream>>>(marginals, lists, d.vocab, L.S, L.slice_len);
    build_kernel<<<dim3((unsigned)d.batch), dim3(256), 0, stream>>>(
        lists, cost, l_ar, d.depth, L.S, d.n_max, (d.flags & BOLE_BUILD_FIXED_BUDGET) ? 1 : 0,
        nn, par, tok, rh, speedup);
    pack_kernel<<<dim3(1), dim3(kPackThreads), 0, stream>>>(nn, par, tok, rh, d.batch, d.n_max,
                                                          node_offsets, parent, token, rho);
    return hipGetLastError();
}

}  // namespace bole
