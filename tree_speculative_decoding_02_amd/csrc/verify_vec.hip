// verify_vec.hip - matrix-core tree verification for bf16 factors and per-channel
// (vector) gates, the GLA / RWKV-6 layout: H_i = diag(g_i) H_parent(i) + k_i v_i^T.
//
// Closed form of the Bole summary page, section 1 ("Tree-Structured Closed Form"), with
// the diagonal transition kept per channel. With LG_i[c] = sum over path(i) of
// log2 g_m[c]:
//     o_i = H_0^T (2^{LG_i} * q_i) + sum_{j on path(i)} w_ij v_j,
//     w_ij = sum_c q_i[c] k_j[c] 2^{LG_i[c] - LG_j[c]}.
// The decay no longer factors out of the products as a row scale, so:
//  - the H_0 term runs on bf16 matrix cores with the decayed query 2^{LG_i} * q_i
//    (fp32, split hi + lo) as the A operand and H_0 (split hi + lo) as the B operand:
//    three products per tile (hi.hi, hi.lo, lo.hi);
//  - the intra-tree term runs on matrix cores too when the tree's LG range allows it
//    (w_ij as the dot product of q_i 2^{LG_i - M} and k_j 2^{M - LG_j}, M the range's
//    midpoint); otherwise each ancestor pair's weight is a 128-channel sum on the vector
//    ALU with exact exponents LG_i - LG_j <= 0, so no factor can overflow.
//
// One 256-thread workgroup per (sequence, head, 64-column group), or, for a verify launch
// short enough to be resident at once, one 512-thread workgroup per two column groups;
// trees of up to 64 nodes; up to 16 layers per launch. Every input is staged through
// registers with plain 16-byte loads issued in the order of use (parent, gate, K, Q
// fragments; H_0 and V once the gate rows have landed), so the H_0 and V loads stay in
// flight while the first phases compute, and each phase waits only for what it reads:
//  1. wavefront 0 builds the topology; the gate and K rows go to LDS;
//  2. gate -> log2 -> root-first cumulative sums LG by pointer doubling across lanes:
//     lane = node, each wavefront holds a slice of the channels in registers, and round
//     r adds the sums held by the node's 2^r-th ancestor, read from its lane
//     (ceil(log2 depth) rounds, no barriers);
//  3. the LG range; pair weights (exact path) or key operands and S tiles (factored
//     path); each wavefront builds its decayed-query operands for one 16-node tile;
//  4. H_0 and V go to LDS, H_0 reusing the space of the LG and K tables;
//  5. H_0 term (v_mfma_f32_16x16x32_bf16, B operands read as 16-byte rows: lane (n, g)
//     takes columns CPL*n ..), the intra term accumulated into the same registers, and
//     the rows stored.
// About 74 KB of LDS at d_k = 128 (two workgroups per CU), 98 KB for a pair.
#include "bole_device.h"
#include "launch.h"
#include "mfma_util.h"

namespace bole {

constexpr int kVecThreads = 256;
// launches of at most this many one-column-group workgroups (two per CU on 256 CUs) take
// the two-group form (see launch_vec_shape)
constexpr uint64_t kVecPairMaxWorkgroups = 512;

// The previous step's tree and accepted path, for LAZY (each layer's prev_k, prev_v and
// prev_gate are its factors).
struct VecLazy {
    const int32_t *parent, *node_offsets, *accepted_idx, *accepted_len;
    int32_t *path_nodes, *tree_status;
    int T, max_path, max_n;
};

// One step of a wavefront-wide running minimum and maximum over DPP lane moves: lanes
// that the move gives no source keep their own values (the identities +inf and -inf).
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ void range_dpp_step(float &mn, float &mx) {
    const int pinf = __builtin_bit_cast(int, __builtin_inff());
    const int ninf = __builtin_bit_cast(int, -__builtin_inff());
    mn = fminf(mn, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                                 pinf, __builtin_bit_cast(int, mn), CTRL, ROW_MASK, 0xf, false)));
    mx = fmaxf(mx, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                                 ninf, __builtin_bit_cast(int, mx), CTRL, ROW_MASK, 0xf, false)));
}

// LAZY: the unit's H_0 slice first takes the previous step's accepted path, with the
// rules and outputs of bole_commit_path (vector gates: H <- diag(g) H + k v^T per path
// node): wavefront 0 validates the path beside the topology, the path factors (gate
// and k rows, the group's v columns) go through the V table's LDS space kStage nodes at
// a time before V needs it, and each thread updates the H_0 rows it holds and writes them
// back, just before they become matrix operands. A unit whose tree of this step is bad or
// empty is committed all the same.
// Layer blockIdx.y of the table; every layer runs the same trees, and the per-tree
// outputs (statuses, path rows) are written by layer 0 only.
// CG = 2 (d_v a multiple of 128): one 512-thread workgroup takes two 64-column groups of a
// unit, so the work that does not depend on the columns (topology, LG, pair weights, query
// and key operands, S tiles) is done once for both; threads 256 h .. 256 h + 255 take
// group h's H_0 rows, V columns and products, and waves w and w + 4 share node tile w.
template <int DK, int DV, bool LAZY, int CG>
__global__ __launch_bounds__(kVecThreads * CG) void verify_vec_kernel(
    const LayerTable lt, const int32_t *__restrict__ parent,
    const int32_t *__restrict__ node_offsets, int32_t *__restrict__ tree_status, int H, int T,
    int U, int max_n, VecLazy lz) {
    constexpr int N = kMaxTree;             // node rows staged (tree nodes; the rest clamped)
    constexpr int NT = kVecThreads * CG;    // threads per workgroup
    constexpr int CW = DV < 64 ? DV : 64;   // state columns per column group
    constexpr int CGW = CW * CG;            // state columns per workgroup
    constexpr int CPL = CW / 16;            // columns per lane in the products
    constexpr int G = DV / CW;              // column groups per unit
    constexpr int GS = G / CG;              // workgroups per unit
    static_assert(CG == 1 || (CG == 2 && G % 2 == 0), "column groups per workgroup");
    constexpr int KT = DK / 32;             // k-steps of the 16x16x32 products
    constexpr int CH = DK / 4;              // channels per lane in the pair weights
    // 16-byte pieces per thread of each staged table
    constexpr int GP = DK / 4, GPT = N * GP / NT;     // gate rows, fp32
    constexpr int KP = DK / 8, KPT = N * KP / NT;     // K rows, bf16
    constexpr int HRG = DK / 8;                       // H_0 slice: 8-row groups
    constexpr int VP = CGW / 8, VPT = N * VP / NT;    // V rows (the workgroup's columns), bf16
    static_assert(GPT >= 1 && KPT >= 1 && VPT >= 1 && HRG * 16 <= kVecThreads, "staging split");
    typedef float hvec __attribute__((ext_vector_type(CPL)));
    typedef __bf16 vvec __attribute__((ext_vector_type(CPL)));
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    // phase A: LG (N x DK fp32) then K (N x DK bf16); phase B: each column group's H_0
    // slice (DK x CW, as bf16 hi and lo tables)
    constexpr int kBig =
        (N * DK + N * DK / 2) > CG * DK * CW ? (N * DK + N * DK / 2) : CG * DK * CW;
    __shared__ __attribute__((aligned(16))) float s_big[kBig];
    __shared__ __attribute__((aligned(16))) __bf16 s_v[N * CGW];  // V rows, the columns
    __shared__ float s_w[N * N];                                   // w_ij at [N i + j]
    __shared__ uint64_t s_mask[N];
    __shared__ int s_anc[6][N];                                    // 2^r-th ancestor (or -1)
    __shared__ int s_info[2];                                      // status, doubling rounds
    __shared__ float s_red[NT / 64][2];                            // per wave: min, max of LG
    __shared__ int s_pinfo[2];                                     // LAZY: path status, length
    __shared__ int s_prow[LAZY ? 64 : 1];                          // LAZY: path rows
    float *s_lg = s_big;
    __bf16 *s_k = reinterpret_cast<__bf16 *>(s_big + N * DK);

    const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
    const int tw = wave & 3;                // node tile of this wavefront's products
    const int hf = tid / kVecThreads;       // column group of this thread within the workgroup
    const int tl = tid - hf * kVecThreads;  // thread index within its column group
    // this thread's column group's H_0 slice: its hi table, then its lo table
    __bf16 *const s_h0g = reinterpret_cast<__bf16 *>(s_big) + hf * 2 * DK * CW;
    int unit, cg;
    if (GS == 1) {
        unit = blockIdx.x;
        cg = 0;
    } else {
        const int slot = blockIdx.x >> 3;
        cg = slot % GS;
        unit = (slot / GS) * 8 + (blockIdx.x & 7);
        if (unit >= U) return;
    }
    const int b = unit / H, h = unit - b * H;
    const int c0 = cg * CGW;
    const bool first = blockIdx.y == 0 && h == 0 && cg == 0;  // writes the per-tree outputs
    const bool writer = tree_status != nullptr && first && tid == 0;
    const bole_layer_t &ly = lt.l[blockIdx.y];
    float *const H0 = ly.H0;  // written only by the lazy commit
    const __bf16 *const q = static_cast<const __bf16 *>(ly.q);
    const __bf16 *const k = static_cast<const __bf16 *>(ly.k);
    const __bf16 *const v = static_cast<const __bf16 *>(ly.v);
    const float *const gate = ly.gate;
    float *const out = ly.out;

    const TreeRange tr = tree_range(node_offsets, b, T, max_n);
    // H_0 slice of this thread's column group: rows 8 hrg .., columns CPL*hn ..
    float *const hu = H0 + (size_t)unit * DK * DV + c0 + hf * CW;
    const int hrg = tl >> 4, hn = tl & 15;

    // ---- LAZY: the previous step's path. Its offsets and length, then (wavefront 0) its
    // parent links and indices; thread t stages chunk t of the first kStage path nodes, a
    // 16-byte piece of a node's gate row, k row or v columns (16 * t bytes into the stage).
    constexpr int kStage = 4;
    constexpr int SGC = DK / 4, SKC = DK / 8, SVC = CGW / 8, CPN = SGC + SKC + SVC;
    constexpr int SB = 16 * CPN;            // stage bytes per path node
    static_assert(!LAZY || (kStage * CPN <= NT && kStage * SB <= N * CGW * 2), "path staging");
    TreeRange ptr = {0, 0, BOLE_TREE_OK};
    int plen_raw = 0, lx = 0, lx2 = 0, lpx = -1, lpp = -1;
    bool plikely = false;
    if constexpr (LAZY) {
        ptr = tree_range(lz.node_offsets, b, lz.T, lz.max_n);
        plen_raw = lz.accepted_len[b];
        plikely = ptr.status == BOLE_TREE_OK && plen_raw > 0 && plen_raw <= lz.max_path &&
                  plen_raw <= ptr.n;
        const int32_t *acc_b = lz.accepted_idx + (size_t)b * lz.max_path;
        if (plikely && tid / CPN < min(kStage, plen_raw)) lx = acc_b[tid / CPN];
        if (plikely && tid / CPN < min(kStage, plen_raw - kStage)) lx2 = acc_b[kStage + tid / CPN];
        if (wave == 0 && ptr.status == BOLE_TREE_OK && ptr.n > 0) {
            lpp = lane < ptr.n ? lz.parent[ptr.lo + lane] : -1;
            if (lane < plen_raw && plen_raw <= lz.max_path) lpx = acc_b[lane];
        }
    }
    // chunk c of path node `row` (a row of the previous step's factors)
    auto path_chunk = [&](int row, int c) -> u32x4 {
        const size_t r = (size_t)row * H + h;
        const void *p =
            c < SGC ? static_cast<const void *>(ly.prev_gate + r * DK + 4 * c)
            : c < SGC + SKC
                ? static_cast<const void *>(static_cast<const __bf16 *>(ly.prev_k) + r * DK +
                                            8 * (c - SGC))
                : static_cast<const void *>(static_cast<const __bf16 *>(ly.prev_v) + r * DV + c0 +
                                            8 * (c - SGC - SKC));
        return *reinterpret_cast<const u32x4 *>(p);
    };
    // the chunks of the first two rounds of kStage path nodes, loaded with the other inputs
    u32x4 pf = {0u, 0u, 0u, 0u}, pf2 = {0u, 0u, 0u, 0u};
    auto prefetch = [&]() {
        if (plikely && tid / CPN < min(kStage, plen_raw))
            pf = path_chunk(ptr.lo + min(max(lx, 0), ptr.n - 1), tid % CPN);
        if (plikely && tid / CPN < min(kStage, plen_raw - kStage))
            pf2 = path_chunk(ptr.lo + min(max(lx2, 0), ptr.n - 1), tid % CPN);
    };
    // wavefront 0: the path checks of the commit, its per-tree outputs, and the path
    // (length, rows) for every thread
    auto validate = [&]() {
        int st = ptr.status, plen = 0, row = -1;
        if (st == BOLE_TREE_OK && ptr.n > 0) {
            const int pn = ptr.n;
            const bool len_ok = plen_raw >= 0 && plen_raw <= lz.max_path;
            const int x = lane < plen_raw ? lpx : -1;
            if (__any(lane < pn && (lpp < -1 || lpp >= lane))) {
                st = BOLE_TREE_BAD_PARENT;
            } else if (!len_ok) {
                st = BOLE_TREE_BAD_PATH;
            } else {
                const int px = __shfl(lpp, (x >= 0 && x < pn) ? x : 0, 64);
                const int prev_raw = __shfl(x, lane > 0 ? lane - 1 : 0, 64);
                const int prev = lane == 0 ? -1 : prev_raw;
                const bool bad = lane < plen_raw && (x < 0 || x >= pn || px != prev);
                if (__any(bad)) st = BOLE_TREE_BAD_PATH;
                else plen = plen_raw;
            }
            row = (st == BOLE_TREE_OK && lane < plen) ? ptr.lo + x : -1;
        } else if (st == BOLE_TREE_OK && plen_raw != 0) {
            st = BOLE_TREE_BAD_PATH;  // a path on an empty tree
        }
        s_prow[lane] = row;
        if (lane == 0) {
            s_pinfo[0] = st;
            s_pinfo[1] = plen;
        }
        if (first) {
            if (lane == 0 && lz.tree_status) lz.tree_status[b] = st;
            if (lz.path_nodes && lane < lz.max_path) lz.path_nodes[(size_t)b * lz.max_path + lane] = row;
        }
    };
    // every thread, after the barrier that publishes the path: the path applied to the
    // H_0 rows this thread holds (rh), kStage nodes at a time, then the rows written back
    auto commit = [&](hvec *rh) {
        const int plen = s_pinfo[1];
        if (plen == 0) return;  // uniform: nothing to commit, H_0 stays as it is
        char *const stage = reinterpret_cast<char *>(s_v);
        for (int m0 = 0; m0 < plen; m0 += kStage) {
            const int mc = min(kStage, plen - m0);
            if (tid / CPN < mc) {
                const u32x4 x = m0 == 0 ? pf
                                : m0 == kStage ? pf2
                                               : path_chunk(s_prow[m0 + tid / CPN], tid % CPN);
                *reinterpret_cast<u32x4 *>(stage + 16 * tid) = x;
            }
            __syncthreads();
            if (hrg < HRG) {
                for (int m = 0; m < mc; ++m) {
                    const char *nb = stage + m * SB;
                    const float4 ga = *reinterpret_cast<const float4 *>(nb + 32 * hrg);
                    const float4 gb = *reinterpret_cast<const float4 *>(nb + 32 * hrg + 16);
                    const bf16x8 kk = *reinterpret_cast<const bf16x8 *>(nb + 4 * DK + 16 * hrg);
                    const vvec vv =
                        *reinterpret_cast<const vvec *>(nb + 6 * DK + 2 * (hf * CW + CPL * hn));
                    const float g8[8] = {ga.x, ga.y, ga.z, ga.w, gb.x, gb.y, gb.z, gb.w};
#pragma unroll
                    for (int e = 0; e < 8; ++e)
#pragma unroll
                        for (int c = 0; c < CPL; ++c)
                            rh[e][c] = g8[e] * rh[e][c] +
                                       static_cast<float>(kk[e]) * static_cast<float>(vv[c]);
                }
            }
            __syncthreads();  // read before the next round, or V, takes the space
        }
        if (hrg < HRG) {
#pragma unroll
            for (int e = 0; e < 8; ++e)
                __builtin_nontemporal_store(
                    rh[e], reinterpret_cast<hvec *>(hu + ((uint32_t)(8 * hrg + e) * DV + CPL * hn)));
        }
    };

    if (tr.status != BOLE_TREE_OK || tr.n == 0) {
        if (writer) tree_status[b] = tr.status;
        if constexpr (LAZY) {
            // nothing to verify: the commit alone
            hvec rh[8];
            if (hrg < HRG) {
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    rh[e] = __builtin_nontemporal_load(reinterpret_cast<const hvec *>(
                        hu + ((uint32_t)(8 * hrg + e) * DV + CPL * hn)));
            }
            prefetch();
            if (wave == 0) validate();
            __syncthreads();
            commit(rh);
        }
        return;
    }
    const int lo = tr.lo, n = tr.n;
    const int last = n - 1;
    const uint32_t rq = (uint32_t)H * DK, rv = (uint32_t)H * DV;
    const __bf16 *qu = q + (size_t)lo * rq + (size_t)h * DK;
    const __bf16 *ku = k + (size_t)lo * rq + (size_t)h * DK;
    const float *gu = gate + (size_t)lo * rq + (size_t)h * DK;
    const __bf16 *vu = v + (size_t)lo * rv + (size_t)h * DV + c0;
    float *ou = out + (size_t)lo * rv + (size_t)h * DV + c0;
    const int n16 = lane & 15, g4 = lane >> 4;
    // pair-weight node and channel quarter (the exact path runs on the first 256 threads)
    const int pi = tl >> 2, psub = tl & 3;
    // LG table: row `row`, 16-byte chunk `ch` (channels 4 ch ..) lies at chunk ch ^ (row mod
    // NCL) of the row, so that 16 lanes reading one chunk of 16 rows fall on distinct banks
    constexpr int NCL = DK / 4;
    auto lgx = [](int row, int ch) { return row * DK + 4 * (ch ^ (row & (NCL - 1))); };

    // ---- issue the loads in order of use (H_0 and V a little later, below). Piece
    // P = tid + NT u of a table with PP pieces per row is row P / PP, piece P % PP (rows
    // past the tree repeat its last row).
    const int p_raw = wave == 0 ? parent[lo + min(lane, last)] : -1;
    u32x4 rg[GPT], rk[KPT], rvv[VPT];
    hvec rh[8];
    // gate and K rows: with several workgroups per unit (GS > 1) each of them reads the
    // unit's rows, so plain loads, which leave the lines in L2 for the others (8-layer
    // stacks of workload 3's shape: verify 105 -> 99 us); one workgroup per unit streams them
    auto row16 = [&](const void *p) -> u32x4 {
        return GS > 1 ? *reinterpret_cast<const u32x4 *>(p)
                      : __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
    };
#pragma unroll
    for (int u = 0; u < GPT; ++u) {
        const int P = tid + NT * u;
        rg[u] = row16(gu + ((uint32_t)min(P / GP, last) * rq + 4 * (P % GP)));
    }
#pragma unroll
    for (int u = 0; u < KPT; ++u) {
        const int P = tid + NT * u;
        rk[u] = row16(ku + ((uint32_t)min(P / KP, last) * rq + 8 * (P % KP)));
    }
    bf16x8 qf[KT];      // Q fragments: row 16*tw + n, channels 32t + 8g .. +7
#pragma unroll
    for (int t = 0; t < KT; ++t)
        qf[t] = load16(qu + ((uint32_t)min(16 * tw + n16, last) * rq + 32 * t + 8 * g4));
    // H_0: thread (hrg, hn) of column group hf loads rows 8 hrg .. 8 hrg + 7 of the group's
    // slice, columns CPL*hn .. (the B-operand rows and columns of one lane); then V. Both
    // are needed last, and are issued once the gate rows have landed (with LAZY, once the
    // first barrier has passed): the gate, K and Q rows that the tree-only phases wait for
    // then reach the workgroup sooner (workload 3: verify 15.6 -> 15.35 us, lazy step
    // 20.8 -> 19.9 us, 8 layers of lazy steps 108.8 -> 105.8 us).
    auto issue_h0_v = [&]() {
        if (hrg < HRG) {
#pragma unroll
            for (int e = 0; e < 8; ++e)
                rh[e] = __builtin_nontemporal_load(
                    reinterpret_cast<const hvec *>(hu + ((uint32_t)(8 * hrg + e) * DV + CPL * hn)));
        }
#pragma unroll
        for (int u = 0; u < VPT; ++u) {
            const int P = tid + NT * u;
            rvv[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(
                vu + ((uint32_t)min(P / VP, last) * rv + 8 * (P % VP))));
        }
    };
    if constexpr (LAZY) prefetch();

    // ---- 1. topology and doubling pointers (wavefront 0); log2 of the gate rows and
    // the K rows to LDS. W needs no clearing: the exact path writes every (node, path
    // node) pair it later reads, and the factored path never reads it.
    if (wave == 0) {
        const WaveTopo topo = wave_topology_p(p_raw, n);
        s_mask[lane] = topo.mask;
        int a = (lane < n && !topo.bad) ? p_raw : -1;
        int rounds = 0;
        for (int r = 0; r < 6 && __any(a >= 0); ++r) {
            s_anc[r][lane] = a;
            rounds = r + 1;
            const int up = __shfl(a, a >= 0 ? a : lane, 64);
            a = a >= 0 ? up : -1;
        }
        if (lane == 0) {
            s_info[0] = topo.bad;
            s_info[1] = rounds;
        }
        if (writer) tree_status[b] = topo.bad;
        if constexpr (LAZY) validate();
    }
#pragma unroll
    for (int u = 0; u < GPT; ++u) {
        const int P = tid + NT * u;
        const float4 x = __builtin_bit_cast(float4, rg[u]);
        *reinterpret_cast<float4 *>(s_lg + lgx(P / GP, P % GP)) =
            make_float4(__builtin_amdgcn_logf(x.x), __builtin_amdgcn_logf(x.y),
                        __builtin_amdgcn_logf(x.z), __builtin_amdgcn_logf(x.w));
    }
    if constexpr (!LAZY) issue_h0_v();
#pragma unroll
    for (int u = 0; u < KPT; ++u) {
        const int P = tid + NT * u;
        *reinterpret_cast<u32x4 *>(s_k + (P / KP) * DK + 8 * (P % KP)) = rk[u];
    }
    __syncthreads();
    if constexpr (LAZY) issue_h0_v();

    if (s_info[0] != BOLE_TREE_OK) {
        if constexpr (LAZY) commit(rh);
        for (int e = tid; e < n * CGW; e += NT)
            ou[(uint32_t)(e / CGW) * rv + (e % CGW)] = __builtin_nanf("");
        return;
    }

    // ---- 2. LG by pointer doubling across lanes: wavefront w holds chunks CPW w .. CPW w
    // + CPW - 1 of every node's row (lane = node) in registers, and round r adds the sums
    // held by each node's 2^r-th ancestor, read from its lane (ds_bpermute): after round r
    // an entry holds the sum over the node's 2^{r+1} nearest path nodes (or its whole
    // path). Every lane reads the sums of the previous round, so no round needs a barrier;
    // each wavefront writes its chunks back, and the range's barrier publishes them.
    constexpr int CPW = NCL / (NT / 64);
    static_assert(NCL % (NT / 64) == 0, "LG chunks per wavefront");
    float4 lv[CPW];
#pragma unroll
    for (int x = 0; x < CPW; ++x)
        lv[x] = *reinterpret_cast<const float4 *>(s_lg + lgx(lane, CPW * wave + x));
    const int rounds = s_info[1];
    for (int r = 0; r < rounds; ++r) {
        const int a = s_anc[r][lane];
        const int src = (a >= 0 ? a : lane) << 2;
        auto pull = [&](float &y) {
            const float t = __builtin_bit_cast(
                float, __builtin_amdgcn_ds_bpermute(src, __builtin_bit_cast(int, y)));
            y = a >= 0 ? y + t : y;
        };
#pragma unroll
        for (int x = 0; x < CPW; ++x) {
            pull(lv[x].x);
            pull(lv[x].y);
            pull(lv[x].z);
            pull(lv[x].w);
        }
    }
#pragma unroll
    for (int x = 0; x < CPW; ++x)
        *reinterpret_cast<float4 *>(s_lg + lgx(lane, CPW * wave + x)) = lv[x];

    // ---- LG range of the tree. With M its midpoint, q_i 2^{LG_i - M} and k_j 2^{M - LG_j}
    // stay within 2^{+-60} when the range is at most 120, and w_ij is then their dot
    // product: the intra term runs on matrix cores. Otherwise (very deep or very strongly
    // decayed trees) each ancestor pair is summed with its exact exponent.
    float lmin = __builtin_inff(), lmax = -__builtin_inff();
    if (lane < n) {
#pragma unroll
        for (int x = 0; x < CPW; ++x) {
            lmin = fminf(lmin, fminf(fminf(lv[x].x, lv[x].y), fminf(lv[x].z, lv[x].w)));
            lmax = fmaxf(lmax, fmaxf(fmaxf(lv[x].x, lv[x].y), fmaxf(lv[x].z, lv[x].w)));
        }
    }
    range_dpp_step<0x111, 0xf>(lmin, lmax);  // row_shr:1
    range_dpp_step<0x112, 0xf>(lmin, lmax);  // row_shr:2
    range_dpp_step<0x114, 0xf>(lmin, lmax);  // row_shr:4
    range_dpp_step<0x118, 0xf>(lmin, lmax);  // row_shr:8
    range_dpp_step<0x142, 0xa>(lmin, lmax);  // row_bcast:15 into rows 1 and 3
    range_dpp_step<0x143, 0xc>(lmin, lmax);  // row_bcast:31 into rows 2 and 3
    if (lane == 63) {  // lane 63 holds the wavefront's minimum and maximum
        s_red[wave][0] = lmin;
        s_red[wave][1] = lmax;
    }
    __syncthreads();
    float lo_lg = s_red[0][0], hi_lg = s_red[0][1];
#pragma unroll
    for (int w = 1; w < NT / 64; ++w) {
        lo_lg = fminf(lo_lg, s_red[w][0]);
        hi_lg = fmaxf(hi_lg, s_red[w][1]);
    }
    const float M = 0.5f * (lo_lg + hi_lg);
    const bool factored = hi_lg - lo_lg <= 120.f && M >= -100.f;

    // ---- 3 (exact path). pair weights w_ij = sum_c q_i[c] k_j[c] 2^{LG_i[c] - LG_j[c]},
    // j on path(i); four lanes per node, CH channels each, summed across the four
    if (!factored && tid < kVecThreads) {
        const uint64_t mi = pi < n ? s_mask[pi] : 0ull;
        bf16x8 qp[CH / 8];  // query channels CH*psub .. of node pi, loaded only on this path
#pragma unroll
        for (int u = 0; u < CH / 8; ++u)
            qp[u] = load16(qu + ((uint32_t)min(pi, last) * rq + CH * psub + 8 * u));
        float qv[CH], li[CH];
#pragma unroll
        for (int u = 0; u < CH / 8; ++u)
#pragma unroll
            for (int e = 0; e < 8; ++e) qv[8 * u + e] = static_cast<float>(qp[u][e]);
        const int ri = min(pi, last);
#pragma unroll
        for (int c = 0; c < CH; c += 4) {
            const float4 x = *reinterpret_cast<const float4 *>(s_lg + lgx(ri, (CH * psub + c) / 4));
            li[c] = x.x;
            li[c + 1] = x.y;
            li[c + 2] = x.z;
            li[c + 3] = x.w;
        }
        uint64_t rest = mi;
        while (rest) {  // the same ancestors for the four lanes of a node
            const int j = __ffsll((unsigned long long)rest) - 1;
            rest &= rest - 1;
            const __bf16 *kj = s_k + j * DK + CH * psub;
            float acc = 0.f;
#pragma unroll
            for (int c = 0; c < CH; c += 8) {
                const bf16x8 kk = *reinterpret_cast<const bf16x8 *>(kj + c);
                const float4 x0 = *reinterpret_cast<const float4 *>(s_lg + lgx(j, (CH * psub + c) / 4));
                const float4 x1 =
                    *reinterpret_cast<const float4 *>(s_lg + lgx(j, (CH * psub + c) / 4 + 1));
                const float lj[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    acc += qv[c + e] * static_cast<float>(kk[e]) *
                           __builtin_amdgcn_exp2f(li[c + e] - lj[e]);
            }
            acc += __shfl_xor(acc, 1, 64);
            acc += __shfl_xor(acc, 2, 64);
            if (psub == 0) s_w[pi * N + j] = acc;
        }
    }
    // query operands of node tile tw: 2^{LG_i[c] - off} q_i[c], split hi + lo, with
    // off = M on the factored path (the H_0 term is scaled back by 2^M) and 0 otherwise
    const float off = factored ? M : 0.f;
    // CG = 2 on the factored path: waves w and w + 4 (same node tile) each build half of
    // the tile's k-steps (column group h: k-steps h KT/2 ..) and hand them to the other
    // through LDS, in the V table (group 0's halves) and the pair-weight table (group
    // 1's), both unused on this path until V is staged
    const bool share = CG == 2 && !LAZY && factored;
    constexpr int KH2 = KT / 2;
    static_assert(CG == 1 || (4 * 2 * KH2 * 64 * 16 <= N * CGW * 2 && 4 * 2 * KH2 * 64 * 16 <= N * N * 4),
                  "operand exchange regions");
    bf16x8 *const x_own = reinterpret_cast<bf16x8 *>(hf == 0 ? static_cast<void *>(s_v) : static_cast<void *>(s_w)) +
                          tw * 2 * KH2 * 64;
    const bf16x8 *const x_other =
        reinterpret_cast<const bf16x8 *>(hf == 0 ? static_cast<void *>(s_w) : static_cast<void *>(s_v)) +
        tw * 2 * KH2 * 64;
    bf16x8 ah[KT], al[KT];
    {
        const int qi = min(16 * tw + n16, last);
#pragma unroll
        for (int t = 0; t < KT; ++t) {
            if (share && (t / KH2) != hf) continue;  // the partner's k-step
            const float4 x0 = *reinterpret_cast<const float4 *>(s_lg + lgx(qi, 8 * t + 2 * g4));
            const float4 x1 = *reinterpret_cast<const float4 *>(s_lg + lgx(qi, 8 * t + 2 * g4 + 1));
            const float lq[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                __bf16 xh, xl;
                split_bf16(static_cast<float>(qf[t][e]) * __builtin_amdgcn_exp2f(lq[e] - off), xh, xl);
                ah[t][e] = xh;
                al[t][e] = xl;
            }
            if (share) {
                x_own[(2 * (t % KH2)) * 64 + lane] = ah[t];
                x_own[(2 * (t % KH2) + 1) * 64 + lane] = al[t];
            }
        }
    }
    // ---- 3 (factored path). S^T tiles (jt, it = tw) = B_jt . A_it^T over channels, with
    // B_j = k_j 2^{M - LG_j} (split hi + lo; three products), masked to ancestors. Their
    // accumulator layout (lane (n, g) holds j = 16jt + 4g + r for node i = 16it + n) is the
    // A operand of W.V over the ancestor tile pair (2p, 2p+1): contraction index 8g + e
    // stands for node 32p + 4g + e (e < 4) or 32p + 16 + 4g + e - 4 (e >= 4).
    bf16x8 wh[2], wl[2];
    if (factored) {
        // B_j = k_j 2^{M - LG_j}, split hi + lo once per entry, into two bf16 tables that
        // take the LG table's space once every wavefront has read LG for its query
        // operands. Their 16-byte chunks are swizzled by row (chunk ^ row mod NCH), so the
        // tile reads below (16 rows, one chunk each) fall on distinct banks.
        constexpr int NCH = DK / 8;
        typedef __bf16 b4 __attribute__((ext_vector_type(4)));
        __bf16 *s_bh = reinterpret_cast<__bf16 *>(s_big);
        __bf16 *s_bl = s_bh + N * DK;
        float4 lgv[GPT];  // LG entries of this thread's key factors: row P / GP, chunk P % GP
#pragma unroll
        for (int u = 0; u < GPT; ++u) {
            const int P = tid + NT * u;
            lgv[u] = *reinterpret_cast<const float4 *>(s_lg + lgx(P / GP, P % GP));
        }
        __syncthreads();
        if (share) {
#pragma unroll
            for (int t = 0; t < KT; ++t) {
                if ((t / KH2) == hf) continue;
                ah[t] = x_other[(2 * (t % KH2)) * 64 + lane];
                al[t] = x_other[(2 * (t % KH2) + 1) * 64 + lane];
            }
        }
#pragma unroll
        for (int u = 0; u < GPT; ++u) {
            const int P = tid + NT * u;
            const int row = P / GP, c = 4 * (P % GP);
            const b4 kk = *reinterpret_cast<const b4 *>(s_k + row * DK + c);
            const float lg[4] = {lgv[u].x, lgv[u].y, lgv[u].z, lgv[u].w};
            b4 hh, ll;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                __bf16 xh, xl;
                split_bf16(static_cast<float>(kk[e]) * __builtin_amdgcn_exp2f(M - lg[e]), xh, xl);
                hh[e] = xh;
                ll[e] = xl;
            }
            const int at = row * DK + 8 * ((c >> 3) ^ (row & (NCH - 1))) + (c & 7);
            *reinterpret_cast<b4 *>(s_bh + at) = hh;
            *reinterpret_cast<b4 *>(s_bl + at) = ll;
        }
        __syncthreads();
        const uint64_t mi = s_mask[16 * tw + n16];
        float w[4][4];
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) {
            f32x4 st = {0.f, 0.f, 0.f, 0.f};
            // CG = 2: each of waves w and w + 4 takes one ancestor tile pair (column group
            // h: tiles 2h and 2h + 1), the other's weights come through LDS
            if (jt <= tw && !(share && (jt >> 1) != hf)) {
                const int j = 16 * jt + n16;
#pragma unroll
                for (int t = 0; t < KT; ++t) {
                    const int at = j * DK + 8 * ((4 * t + g4) ^ (j & (NCH - 1)));
                    const bf16x8 bh = load16(s_bh + at), bl = load16(s_bl + at);
                    st = mfma16_bf16(bh, ah[t], st);
                    st = mfma16_bf16(bh, al[t], st);
                    st = mfma16_bf16(bl, ah[t], st);
                }
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int j = 16 * jt + 4 * g4 + r;
                w[jt][r] = (jt <= tw && ((mi >> j) & 1ull)) ? st[r] : 0.f;
            }
        }
#pragma unroll
        for (int p = 0; p < 2; ++p)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                __bf16 xh, xl;
                split_bf16(e < 4 ? w[2 * p][e] : w[2 * p + 1][e - 4], xh, xl);
                wh[p][e] = xh;
                wl[p][e] = xl;
            }
        if (share && 2 * hf <= tw) {
            // this wave's pair into the pair-weight table (its operand halves there were
            // read before the last barrier)
            bf16x8 *const wx = reinterpret_cast<bf16x8 *>(s_w) + wave * 128;
#pragma unroll
            for (int p = 0; p < 2; ++p)
                if (p == hf) {
                    wx[lane] = wh[p];
                    wx[64 + lane] = wl[p];
                }
        }
    }
    __syncthreads();  // LG and K are dead: the H_0 slice takes their space
    if (share && 2 * (1 - hf) <= tw) {
        const bf16x8 *const wx = reinterpret_cast<const bf16x8 *>(s_w) + (wave ^ 4) * 128;
#pragma unroll
        for (int p = 0; p < 2; ++p)
            if (p != hf) {
                wh[p] = wx[lane];
                wl[p] = wx[64 + lane];
            }
    }
    if constexpr (LAZY) commit(rh);

    // ---- 4. H_0 and V to LDS. H_0 is split hi + lo once here, into two bf16 tables in
    // B-operand order: the 16 bytes at [(rg CPL + c) 16 + n] hold rows 8rg .. 8rg + 7 of
    // column CPL*n + c, so each product reads its operands with one 16-byte load per lane
    // (the 16 lanes of a row group contiguous) and splits nothing.
    if (hrg < HRG) {
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            bf16x8 hh, ll;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                __bf16 xh, xl;
                split_bf16(rh[e][c], xh, xl);
                hh[e] = xh;
                ll[e] = xl;
            }
            const int at = ((hrg * CPL + c) * 16 + hn) * 8;
            *reinterpret_cast<bf16x8 *>(s_h0g + at) = hh;
            *reinterpret_cast<bf16x8 *>(s_h0g + DK * CW + at) = ll;
        }
    }
#pragma unroll
    for (int u = 0; u < VPT; ++u) {
        const int P = tid + NT * u;
        *reinterpret_cast<u32x4 *>(s_v + (P / VP) * CGW + 8 * (P % VP)) = rvv[u];
    }
    __syncthreads();

    // ---- 5. H_0 term for node tile tw and this thread's column group, then the intra
    // term, then the rows
    f32x4 acc[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < KT; ++t) {
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            const int at = (((4 * t + g4) * CPL + c) * 16 + n16) * 8;
            const bf16x8 bh = load16(s_h0g + at), bl = load16(s_h0g + DK * CW + at);
            acc[c] = mfma16_bf16(ah[t], bh, acc[c]);
            acc[c] = mfma16_bf16(ah[t], bl, acc[c]);
            acc[c] = mfma16_bf16(al[t], bh, acc[c]);
        }
    }
    if (factored) {
        const float sc = __builtin_amdgcn_exp2f(M);
#pragma unroll
        for (int c = 0; c < CPL; ++c) acc[c] *= sc;
        // W.V: V operand for column tile c, element e = V[32p + j(e)][CPL*n + c]
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            if (2 * p > tw) break;
            bf16x8 vb[CPL];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int j = 32 * p + (e < 4 ? 4 * g4 + e : 12 + 4 * g4 + e);
                const vvec x = *reinterpret_cast<const vvec *>(s_v + j * CGW + hf * CW + CPL * n16);
#pragma unroll
                for (int c = 0; c < CPL; ++c) vb[c][e] = x[c];
            }
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
                acc[c] = mfma16_bf16(wh[p], vb[c], acc[c]);
                acc[c] = mfma16_bf16(wl[p], vb[c], acc[c]);
            }
        }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int i = 16 * tw + 4 * g4 + r;
        if (i >= n) continue;
        uint64_t rest = factored ? 0ull : s_mask[i];
        while (rest) {
            const int j = __ffsll((unsigned long long)rest) - 1;
            rest &= rest - 1;
            const float w = s_w[i * N + j];
            const vvec vv = *reinterpret_cast<const vvec *>(s_v + j * CGW + hf * CW + CPL * n16);
#pragma unroll
            for (int c = 0; c < CPL; ++c) acc[c][r] += w * static_cast<float>(vv[c]);
        }
        hvec o;
#pragma unroll
        for (int c = 0; c < CPL; ++c) o[c] = acc[c][r];
        __builtin_nontemporal_store(
            o, reinterpret_cast<hvec *>(ou + ((uint32_t)i * rv + hf * CW + CPL * n16)));
    }
}

bool verify_vec_applies(const bole_dims_t &d, const void *H0, const void *q, const void *k,
                        const void *v, const void *gate, const void *out) {
    if (d.flags & BOLE_FLAG_FORCE_GENERIC) return false;
    if (d.factor_dtype != BOLE_DTYPE_BF16 || d.gate_kind != BOLE_GATE_VECTOR) return false;
    if (d.d_k != 64 && d.d_k != 128) return false;
    if (d.d_v != 32 && d.d_v != 64 && d.d_v != 128 && d.d_v != 256) return false;
    const uintptr_t a = reinterpret_cast<uintptr_t>(H0) | reinterpret_cast<uintptr_t>(q) |
                        reinterpret_cast<uintptr_t>(k) | reinterpret_cast<uintptr_t>(v) |
                        reinterpret_cast<uintptr_t>(gate) | reinterpret_cast<uintptr_t>(out);
    if (a % 16 != 0) return false;
    const uint64_t row_elems = (uint64_t)d.heads * (uint64_t)(d.d_k > d.d_v ? d.d_k : d.d_v);
    if (row_elems * kMaxTree >= (1ull << 31)) return false;
    const uint64_t groups = d.d_v > 64 ? (uint64_t)d.d_v / 64 : 1;
    return ((uint64_t)d.batch * (uint64_t)d.heads + 8) * groups < (1ull << 30);
}

// nl <= kLayersPerLaunch layers sharing their trees, one launch (blockIdx.y = layer);
// lz: the lazy commit (H0 is then written), else nullptr (H0 is only read)
template <int DK, int DV>
static void launch_vec_shape(const bole_layer_t *layers, int nl, const int32_t *parent,
                             const int32_t *node_offsets, const bole_dims_t &d,
                             int32_t *tree_status, hipStream_t stream, const VecLazy *lz) {
    constexpr int G = DV < 64 ? 1 : DV / 64;
    const unsigned U = (unsigned)d.batch * (unsigned)d.heads;
    LayerTable lt = {};
    for (int l = 0; l < nl; ++l) lt.l[l] = layers[l];
    const int mn = max_tree_nodes(d.flags);
    const VecLazy none = {};
    // Verify takes two column groups per workgroup when the launch is short enough for all
    // of its one-group workgroups to be resident at once (two per CU): each workgroup's
    // chain is then the launch's time, and the pair does its column-independent work once
    // (workload 3: 17.8 -> 16.3 us). Longer launches keep one group per workgroup: two
    // workgroups per CU overlap one unit's products with another's loads, which one
    // 8-wavefront workgroup does less (8-layer stacks 2-3% slower as pairs), and so does
    // the lazy form, whose commit rounds the pair does not shorten (0.4 us slower).
    const unsigned slots1 = G == 1 ? U : ((U + 7) / 8) * 8 * G;
    if constexpr (G % 2 == 0) {
        if (!lz && (uint64_t)slots1 * (uint64_t)nl <= kVecPairMaxWorkgroups) {
            constexpr int GS = G / 2;
            const dim3 grid(GS == 1 ? U : ((U + 7) / 8) * 8 * GS, (unsigned)nl);
            verify_vec_kernel<DK, DV, false, 2><<<grid, dim3(2 * kVecThreads), 0, stream>>>(
                lt, parent, node_offsets, tree_status, d.heads, d.total_nodes, (int)U, mn, none);
            return;
        }
    }
    const dim3 grid(slots1, (unsigned)nl);
    if (lz)
        verify_vec_kernel<DK, DV, true, 1><<<grid, dim3(kVecThreads), 0, stream>>>(
            lt, parent, node_offsets, tree_status, d.heads, d.total_nodes, (int)U, mn, *lz);
    else
        verify_vec_kernel<DK, DV, false, 1><<<grid, dim3(kVecThreads), 0, stream>>>(
            lt, parent, node_offsets, tree_status, d.heads, d.total_nodes, (int)U, mn, none);
}

static hipError_t launch_vec(const bole_layer_t *layers, int nl, const int32_t *parent,
                             const int32_t *node_offsets, const bole_dims_t &d,
                             int32_t *tree_status, hipStream_t stream, const VecLazy *lz) {
#define BOLE_VEC_CASE(DKV, DVV)                                                                \
    if (d.d_k == DKV && d.d_v == DVV) {                                                         \
        launch_vec_shape<DKV, DVV>(layers, nl, parent, node_offsets, d, tree_status, stream, lz); \
        return hipGetLastError();                                                               \
    }
    BOLE_VEC_CASE(64, 32) BOLE_VEC_CASE(64, 64) BOLE_VEC_CASE(64, 128) BOLE_VEC_CASE(64, 256)
    BOLE_VEC_CASE(128, 32) BOLE_VEC_CASE(128, 64) BOLE_VEC_CASE(128, 128) BOLE_VEC_CASE(128, 256)
#undef BOLE_VEC_CASE
    return hipErrorInvalidValue;
}

hipError_t launch_verify_vec(const bole_layer_t *layers, int nl, const int32_t *parent,
                             const int32_t *node_offsets, const bole_dims_t &d,
                             int32_t *tree_status, hipStream_t stream) {
    return launch_vec(layers, nl, parent, node_offsets, d, tree_status, stream, nullptr);
}

bool verify_vec_lazy_applies(const bole_dims_t &d, const bole_dims_t &pd, const bole_layer_t &y) {
    if (!verify_vec_applies(d, y.H0, y.q, y.k, y.v, y.gate, y.out)) return false;
    // the previous step's factors: same layout and shapes, 16-byte rows
    if (pd.factor_dtype != d.factor_dtype || pd.gate_kind != d.gate_kind || pd.d_k != d.d_k ||
        pd.d_v != d.d_v || pd.heads != d.heads || pd.batch != d.batch)
        return false;
    const uintptr_t a = reinterpret_cast<uintptr_t>(y.prev_k) |
                        reinterpret_cast<uintptr_t>(y.prev_v) |
                        reinterpret_cast<uintptr_t>(y.prev_gate);
    return a % 16 == 0;
}

hipError_t launch_verify_vec_lazy(const bole_layer_t *layers, int nl, const PrevPath &prev,
                                  const bole_dims_t &pd, const int32_t *parent,
                                  const int32_t *node_offsets, const bole_dims_t &d,
                                  int32_t *tree_status, hipStream_t stream) {
    VecLazy lz;
    lz.parent = prev.parent;
    lz.node_offsets = prev.node_offsets;
    lz.accepted_idx = prev.accepted_idx;
    lz.accepted_len = prev.accepted_len;
    lz.path_nodes = prev.path_nodes;
    lz.tree_status = prev.tree_status;
    lz.T = pd.total_nodes;
    lz.max_path = pd.max_path;
    lz.max_n = max_tree_nodes(pd.flags);
    return launch_vec(layers, nl, parent, node_offsets, d, tree_status, stream, &lz);
}

}  // namespace bole
