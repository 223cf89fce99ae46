// verify_mfma.hip - matrix-core tree verification for bf16 factors and scalar gates
// (the Mamba-2 layout).
//
// It evaluates the closed form of the Bole summary page, section 1 ("Tree-Structured
// Closed Form"), for every node of a tree at once:
//     O = diag(2^{L}) (Q H_0) + W V,   W_ij = (q_i . k_j) 2^{L_i - L_j} [j on path(i)]
// L_i is the root-first sum of log2 a over path(i). Only per-node factors are read
// (section 2, "Token-Level Factor Encoding"); no per-node state exists anywhere.
//
// Trees of 1..32 nodes take one wavefront per sequence, head and column group (64 state
// columns; 32 in short launches); trees of 33..64 nodes take
// two wavefronts that split H_0's rows. A batch that may hold larger trees runs both in
// one fused launch, packed (four small-tree or two large-tree units per workgroup) when
// the head count allows; each launch covers up to 16 layers that share the trees
// (blockIdx.y = layer). The LAZY instantiations first apply the previous step's
// accepted path to H_0 (section 2's restore) and write it back, in the same pass over
// H_0: each unit is committed by the body (one wavefront, or the row split) that
// verifies its tree.
// H_0 goes from HBM straight into MFMA operand registers with
// row-contiguous 16-byte loads, so a wavefront needs only 12 KB of LDS (K and V) and
// eight of them fit on a CU: the whole benchmark batch is in flight at once. fp32
// operands (H_0, W) are split into bf16 hi + lo (two products, about 16 mantissa bits),
// and non-ancestors are masked by select, never by multiplication, so pairs whose decay
// factor overflows can never produce NaN. Topology and the base-2 cumulative decay are
// rebuilt by each wavefront on its own 64 lanes (lane = node), with no barrier.
#include "bole_device.h"
#include "launch.h"
#include "mfma_util.h"

namespace bole {

// Trees of 1..32 nodes (and the status of every tree except those of 33..64 nodes, which
// the two-wavefront body below takes): one wavefront per (sequence, head, 64-column
// group) covers the tree's 32 node rows as two 16-node tiles. 16x16 matrix-core tiles
// throughout: lane = (n, g) with n = lane % 16, g = lane / 16.
//
// H_0 term, all v_mfma_f32_16x16x32_bf16. The H_0 slice is loaded straight into
// registers with row-contiguous loads: load s = 8t + e gives lane (n, g) row
// 32t + 8g + e, columns CPL n .. CPL n + CPL - 1 (CPL = 4 for 64 columns, 16 bytes; 2 for
// 32), and one load instruction covers 4 full rows of the group. Over the 8 loads of
// k-step t, lane (n, g) then holds rows 32t + 8g .. +7 of each of its columns: exactly
// the B operand of a 16x16x32 product whose output column n stands for state column
// CPL n + c. H_0 never goes through LDS. It is split bf16 hi + lo (two
// products, about 16 mantissa bits); the A operand is the bf16 Q fragment of the same
// k-step, shared with the intra-tree term.
//
// Intra-tree term on the same products:
//  - S^T tile (jt, it) = K_jt . Q_it^T over d_k, for every ancestor tile jt <= it; K
//    comes from LDS (16-byte pieces XOR-swizzled by row so the fragment reads are
//    conflict-free), Q from registers;
//  - the accumulator layout (lane (n, g) holds j = 16jt + 4g + r for node i = 16it + n)
//    is used in place as the A operand of W.V over a pair of ancestor tiles (2p, 2p+1):
//    contraction index 8g + e stands for node 32p + 4g + e (e < 4) or
//    32p + 16 + 4g + e - 4 (e >= 4); V is gathered from LDS in the same order;
//  - W = S * 2^{L_i - L_j} on ancestors, selected to 0 elsewhere, split bf16 hi + lo.
// Both terms land in one accumulator layout: lane (n, g) holds node 16it + 4g + r,
// state columns CPL n .. across its CPL tiles, stored as one write per row.
// Read-once and write-once streams carry the non-temporal cache policy.
// The previous step's tree and accepted path, for the lazy-commit form (LAZY): the kernel
// first applies that path (with the layer's prev_k, prev_v, prev_gate) to H_0 in
// registers and writes the committed state back, then verifies this step's tree against it.
struct LazyCommit {
    const int32_t *parent, *node_offsets, *accepted_idx, *accepted_len;
    int32_t *path_nodes, *tree_status;
    int T, max_path, max_n;
};

// Layer blockIdx.y of the table; every layer runs the same trees. Per-tree outputs
// (statuses, path rows) are written by layer 0 only.
// CWM: the most state columns a workgroup (a unit's column group) takes, 64, or 32 for
// launches too short to fill the chip (two column groups per unit at d_v = 64)
template <int DK, int DV, int CWM>
constexpr int ksplit_smem_bytes();
template <int DK, int DV, int CWM>
constexpr int ksplit_lazy_smem_elems();
template <int DK, int DV, bool LAZY, int CWM>
__device__ __forceinline__ void ksplit_body(const bole_layer_t, const int32_t *, const int32_t *,
                                            int32_t *, int, int, int, int, char *, int, int,
                                            const LazyCommit &, __bf16 *, const TreeRange *);

// Packed fused launch (FUSED, NW = 4 or 8 slots, a head count divisible by NW): wavefront
// slots are dealt to the units in sequence order, two to each unit whose tree has 33..64
// nodes and one to every other unit, NW slots per workgroup. Each sequence's units take a
// multiple of NW slots, so a workgroup holds units of one sequence only: NW one-wavefront
// units or NW / 2 row-split units. Every wavefront finds its slot's sequence from the tree offsets
// of all sequences (a running count of large trees, one ballot per 64 sequences); the
// grid is sized for the case of every tree large, and workgroups past the last slot exit.
struct PackSlot {
    int b;          // sequence, -1 past the last slot
    int r;          // slot within the sequence's slots
    bool large;     // a tree of 33..64 nodes (two slots per unit)
    TreeRange tr;   // the sequence's tree range, as tree_range() gives it
};

__device__ __forceinline__ PackSlot pack_locate(const int32_t *__restrict__ node_offsets, int B,
                                                int H, int T, int max_n, int s) {
    const int lane = lane_id();
    int base = 0;   // slots of the sequences before this chunk of 64
    for (int c0 = 0; c0 < B; c0 += 64) {
        const int b = c0 + lane;
        int lo = 0, hi = 0;
        if (b < B) {
            lo = node_offsets[b];
            hi = node_offsets[b + 1];
        }
        const bool bad = lo < 0 || hi < lo || hi > T || hi - lo > max_n;
        const uint64_t lm = __ballot(b < B && !bad && hi - lo > 32);
        // first slot of sequence b: H per sequence before it, H more per large one
        const int before = (int)__builtin_amdgcn_mbcnt_hi(
            (uint32_t)(lm >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)lm, 0u));
        const int start = base + H * (lane + before);
        const int total = H * (min(64, B - c0) + (int)__popcll(lm));
        if (s < base + total) {
            // the sequences starting at or before s are a prefix of the chunk's lanes
            const int bl = (int)__popcll(__ballot(b < B && start <= s)) - 1;
            PackSlot p;
            p.b = c0 + bl;
            p.r = s - __builtin_amdgcn_readlane(start, bl);
            p.large = (lm >> bl) & 1;
            p.tr.lo = __builtin_amdgcn_readlane(lo, bl);
            p.tr.n = __builtin_amdgcn_readlane(hi, bl) - p.tr.lo;
            p.tr.status = __builtin_amdgcn_readlane(bad ? (int)BOLE_TREE_BAD_SIZE : (int)BOLE_TREE_OK, bl);
            return p;
        }
        base += total;
    }
    PackSlot p;
    p.b = -1;
    p.r = 0;
    p.large = false;
    p.tr = {0, 0, BOLE_TREE_OK};
    return p;
}

// FUSED: every tree size in one launch, for a caller without a budget of 32 nodes (with
// LAZY, each body also commits the units whose trees it verifies). Each
// unit of the workgroup has two wavefronts and an LDS region of its own: a tree of 33..64
// nodes takes the row-split body (below) on both, one of up to 32 nodes the one-wavefront
// body on the first (the second exits); both leave at once, and wave-uniformly, for the
// trees they do not take. With NW = 2 a workgroup of four wavefronts takes heads 2j and
// 2j + 1 of one sequence (so one tree, and the row-split barriers of both units match).
// FUSED with NW = 4 or 8: the packed launch (above), 64 NW threads.
// CWM: the most state columns a workgroup takes (64, or 32 for two column groups per unit
// at d_v = 64).
// NW > 1 (one column group per unit, not FUSED): a workgroup of NW wavefronts takes NW
// consecutive units, heads NW j .. NW j + NW - 1 of a sequence, one per wavefront, each with
// its own LDS. A node's q, k, v and out rows of neighbouring heads are adjacent in the
// token-major layout, so the group's row pieces form runs NW times as long, requested
// together by one CU.
template <int DK, int DV, bool LAZY, bool FUSED, int NW, int CWM>
__global__ __launch_bounds__(FUSED && NW <= 2 ? 128 * NW : 64 * NW, 2) void verify_mfma_tree_kernel(
    const LayerTable lt, const int32_t *__restrict__ parent,
    const int32_t *__restrict__ node_offsets, int32_t *__restrict__ tree_status, int H, int T,
    int U, int max_n, LazyCommit lc) {
    constexpr int NN = 32;                  // node rows staged
    constexpr int NT = 2;                   // 16-node tiles
    constexpr int CW = DV < CWM ? DV : CWM; // state columns per workgroup
    constexpr int CPL = CW / 16;            // columns per lane: 4 or 2
    constexpr int G = DV / CW;              // column groups per unit
    constexpr int KT = DK / 32;             // k-steps of the bf16 products
    constexpr int HS = DK / 4;              // 16-byte H_0 loads per lane (4 rows each)
    constexpr int PPR = DK / 8;             // 16-byte pieces per K row
    constexpr int VPR = CW / 8;             // 16-byte pieces per V row (of this group's columns)
    typedef float hvec __attribute__((ext_vector_type(CPL)));
    typedef __bf16 vvec __attribute__((ext_vector_type(CPL)));
    static_assert(NW == 1 || G == 1, "unit groups: one column group per unit");
    constexpr bool PACK = FUSED && NW >= 4;
    static_assert(!FUSED || NW <= 2 || NW == 4 || NW == 8, "fused unit groups: two units, or packed");
    static_assert(!PACK || G == 1, "packed launch: one column group per unit");
    // K rows: piece p of row j at slot j*PPR + (p ^ j%PPR); V rows of the group's columns,
    // row j at [CW j]; lazy commit: k rows and v rows (group columns) of up to kLazyStage
    // path nodes. FUSED: K and V in the buffer the row-split body uses.
    constexpr int kLazyStage = LAZY ? 8 : 1;
    static_assert(NN * PPR * 16 + NN * CW * 2 <= ksplit_smem_bytes<DK, DV, CWM>(), "fused LDS region");
    // PACK: NW / 2 row-split regions, or NW one-wavefront regions of half the size
    static_assert(2 * (NN * PPR * 16 + NN * CW * 2) == ksplit_smem_bytes<DK, DV, CWM>(), "packed regions");
    constexpr int kFusedBytes = FUSED ? (PACK ? NW / 2 : NW) * ksplit_smem_bytes<DK, DV, CWM>() : 16;
    __shared__ __align__(16) char s_fused[kFusedBytes];
    __shared__ bf16x8 s_k_own[FUSED ? 1 : NW * NN * PPR];
    __shared__ __bf16 s_v_own[FUSED ? 8 : NW * NN * CW];
    __shared__ __bf16 s_pk_all[NW * kLazyStage * DK], s_pv_all[NW * kLazyStage * CW];
    // FUSED and LAZY: the row-split body's path staging, one region per wavefront
    __shared__ __align__(16) __bf16
        s_lzk[FUSED && LAZY ? (PACK ? NW : 2 * NW) * ksplit_lazy_smem_elems<DK, DV, CWM>() : 8];
    // this wavefront's unit of the group (FUSED, not packed: two wavefronts per unit)
    const int wv = NW > 1 ? __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> (FUSED && !PACK ? 7 : 6))) : 0;
    char *const s_unit = s_fused + (PACK ? wv * (ksplit_smem_bytes<DK, DV, CWM>() / 2)
                                        : FUSED ? wv * ksplit_smem_bytes<DK, DV, CWM>() : 0);
    bf16x8 *const s_k = FUSED ? reinterpret_cast<bf16x8 *>(s_unit) : s_k_own + wv * NN * PPR;
    __bf16 *const s_v = FUSED ? reinterpret_cast<__bf16 *>(s_unit + NN * PPR * 16)
                              : s_v_own + wv * NN * CW;
    __bf16 *const s_pk = s_pk_all + wv * kLazyStage * DK;
    __bf16 *const s_pv = s_pv_all + wv * kLazyStage * CW;
    const bole_layer_t &ly = lt.l[blockIdx.y];
    PackSlot ps = {0, 0, false, {0, 0, BOLE_TREE_OK}};
    if constexpr (PACK) {
        ps = pack_locate(node_offsets, U / H, H, T, max_n, NW * (int)blockIdx.x + wv);
        if (ps.b < 0) return;  // past the last slot: the whole workgroup
        if (ps.large) {
            ksplit_body<DK, DV, LAZY, CWM>(ly, parent, node_offsets, tree_status, H, T, U, max_n,
                                      s_fused + (wv >> 1) * ksplit_smem_bytes<DK, DV, CWM>(),
                                      ps.b * H + (ps.r >> 1), ps.r & 1, lc,
                                      LAZY ? s_lzk + wv * ksplit_lazy_smem_elems<DK, DV, CWM>() : nullptr,
                                      &ps.tr);
            return;
        }
    } else if constexpr (FUSED) {
        ksplit_body<DK, DV, LAZY, CWM>(ly, parent, node_offsets, tree_status, H, T, U, max_n, s_unit,
                                  NW * (int)blockIdx.x + wv, (int)((threadIdx.x >> 6) & 1), lc,
                                  LAZY ? s_lzk + (threadIdx.x >> 6) * ksplit_lazy_smem_elems<DK, DV, CWM>()
                                       : nullptr, nullptr);
        if (threadIdx.x & 64) return;  // the second wavefront of each unit
    }
    float *const H0 = ly.H0;                // written only by the lazy commit
    const __bf16 *const q = static_cast<const __bf16 *>(ly.q);
    const __bf16 *const k = static_cast<const __bf16 *>(ly.k);
    const __bf16 *const v = static_cast<const __bf16 *>(ly.v);
    const float *const gate = ly.gate;
    float *const out = ly.out;

    const int lane = lane_id();
    const int n16 = lane & 15, g = lane >> 4;
    int unit, cg;
    if (PACK) {
        unit = ps.b * H + ps.r;
        cg = 0;
    } else if (G == 1) {
        unit = NW * (int)blockIdx.x + wv;
        if (unit >= U) return;
        cg = 0;
    } else {
        const int slot = blockIdx.x >> 3;
        cg = slot % G;
        unit = (slot / G) * 8 + (blockIdx.x & 7);
        if (unit >= U) return;
    }
    const int b = unit / H, h = unit - b * H;
    const int c0 = cg * CW;
    const bool first = blockIdx.y == 0 && h == 0 && cg == 0;  // writes the per-tree outputs
    const bool writer = tree_status != nullptr && first && lane == 0;

    const TreeRange tr = PACK ? ps.tr : tree_range(node_offsets, b, T, max_n);
    bool do_verify = true;
    if (tr.status != BOLE_TREE_OK) {
        if (writer) tree_status[b] = tr.status;
        do_verify = false;
    } else if (tr.n > 32) {
        // the row-split body's, which in the lazy form also commits the unit's previous
        // path, in the same pass over H_0
        if (LAZY) return;
        do_verify = false;
    } else if (tr.n == 0) {
        if (writer) tree_status[b] = BOLE_TREE_OK;
        do_verify = false;
    }
    // the previous step's path: plausible from its length and offsets alone (validated
    // below, once its parent links and indices are in)
    TreeRange ptr = {0, 0, BOLE_TREE_OK};
    int plen_raw = 0;
    bool plikely = false;
    if constexpr (LAZY) {
        ptr = tree_range(lc.node_offsets, b, lc.T, lc.max_n);
        plen_raw = lc.accepted_len[b];
        plikely = ptr.status == BOLE_TREE_OK && plen_raw > 0 && plen_raw <= lc.max_path &&
                  plen_raw <= ptr.n;
    }
    if (!LAZY && !do_verify) return;
    const int lo = do_verify ? tr.lo : 0, n = do_verify ? tr.n : 1;
    const int last = n - 1;
    const uint32_t rq = (uint32_t)H * DK, rv = (uint32_t)H * DV;
    const __bf16 *qu = q + (size_t)lo * rq + (size_t)h * DK;
    const __bf16 *ku = k + (size_t)lo * rq + (size_t)h * DK;
    const __bf16 *vu = v + (size_t)lo * rv + (size_t)h * DV + c0;
    float *ou = out + (size_t)lo * rv + (size_t)h * DV + c0;
    float *hu = H0 + (size_t)unit * DK * DV + c0;

    // ---- 1. issue every load
    // lazy commit, first: the path indices this lane's factor chunks and the validation
    // need (a chunk is 16 bytes of a path node's k row or of its v row's group columns)
    constexpr int LCK = DK / 8, LCV = CW / 8, LCPN = LCK + LCV;  // chunks per path node
    constexpr int LCH = LAZY ? (kLazyStage * LCPN + 63) / 64 : 1;  // chunks per lane
    int lx[LCH];
    int lpx = -1, lpp = -1;  // lane = path position: accepted index; lane = node: parent
    if constexpr (LAZY) {
        const int32_t *acc_b = lc.accepted_idx + (size_t)b * lc.max_path;
#pragma unroll
        for (int u = 0; u < LCH; ++u) {
            const int m = (lane + 64 * u) / LCPN;
            lx[u] = (plikely && m < plen_raw) ? acc_b[m] : 0;
        }
        if (ptr.status == BOLE_TREE_OK && ptr.n > 0) {
            lpp = lane < ptr.n ? lc.parent[ptr.lo + lane] : -1;
            if (lane < plen_raw && plen_raw <= lc.max_path) lpx = acc_b[lane];
        }
    }
    const uint32_t node = (uint32_t)min(lane, last);
    const int p_raw = do_verify ? parent[lo + node] : -1;
    const float g_raw = do_verify ? gate[(size_t)lo * H + h + node * (uint32_t)H] : 1.f;
    // Q fragments of the tiles: row 16it + n, elements 32t + 8g .. +7
    bf16x8 qf[NT][KT];
    // K and V rows go to LDS through registers (plain loads, so every later wait counts
    // exactly what it needs: no LDS instruction has to wait for the H_0 loads). K: load
    // s fills LDS slots 64s .. 64s+63, i.e. rows (64/PPR)s ..; lane l fills slot 64s + l
    // = row j, slot-in-row l % PPR, with piece (l % PPR) ^ (j % PPR). V: lane l of load s
    // takes row (64/VPR)s + l/VPR, piece l % VPR.
    constexpr int KL = NN * PPR / 64, VL = NN * VPR / 64;
    bf16x8 kst[KL], vst[VL];
    // q and k rows: with several column groups per unit (G > 1) every group's workgroup
    // reads them, so plain loads, which leave the lines in L2 for the others
    auto qk16 = [](const __bf16 *p) { return G > 1 ? load16(p) : load16_stream(p); };
    if (do_verify) {
#pragma unroll
        for (int it = 0; it < NT; ++it)
#pragma unroll
            for (int t = 0; t < KT; ++t)
                qf[it][t] = qk16(qu + ((uint32_t)min(16 * it + n16, last) * rq + 32 * t + 8 * g));
#pragma unroll
        for (int u = 0; u < KL; ++u) {
            const int s = u;
            const int j = (64 / PPR) * s + lane / PPR;
            const int pc = (lane % PPR) ^ (j % PPR);
            kst[u] = qk16(ku + ((uint32_t)min(j, last) * rq + 8 * pc));
        }
#pragma unroll
        for (int u = 0; u < VL; ++u) {
            const int s = u;
            const int j = (64 / VPR) * s + lane / VPR;
            vst[u] = load16_stream(vu + ((uint32_t)min(j, last) * rv + 8 * (lane % VPR)));
        }
    }
    // H_0 slice: load s = 8t + e, lane (n, g): row 32t + 8g + e, columns CPL*n ..
    hvec hreg[HS];
    if (do_verify || plikely) {
#pragma unroll
        for (int s = 0; s < HS; ++s)
            hreg[s] = __builtin_nontemporal_load(reinterpret_cast<const hvec *>(
                hu + ((uint32_t)(32 * (s >> 3) + 8 * g + (s & 7)) * DV + CPL * n16)));
    }
    // lazy commit: the factor chunks of the first kLazyStage path nodes, issued behind
    // H_0 (their indices were loaded first) and held in registers until the path is
    // validated; rows clamped into the tree, which the offsets check keeps inside [0, T)
    bf16x8 pf[LCH];
    if constexpr (LAZY) {
        if (plikely) {
            const int mc0 = min(kLazyStage, plen_raw);
#pragma unroll
            for (int u = 0; u < LCH; ++u) {
                const int c = lane + 64 * u;
                const int m = c / LCPN, part = c - m * LCPN;
                if (m < mc0) {
                    const size_t prow = (size_t)(ptr.lo + min(max(lx[u], 0), ptr.n - 1)) * H + h;
                    pf[u] = part < LCK
                                ? load16(static_cast<const __bf16 *>(ly.prev_k) + prow * DK + 8 * part)
                                : load16(static_cast<const __bf16 *>(ly.prev_v) + prow * DV + c0 +
                                         8 * (part - LCK));
                }
            }
        }
    }
    if (do_verify) {
#pragma unroll
        for (int u = 0; u < KL; ++u) s_k[64 * u + lane] = kst[u];
#pragma unroll
        for (int u = 0; u < VL; ++u)
            *reinterpret_cast<bf16x8 *>(s_v + 512 * u + 8 * lane) = vst[u];
    }

    // ---- lazy commit: validate the previous path, stage its factors, update H_0 in
    // registers, write it back (same rules and outputs as bole_commit_path)
    if constexpr (LAZY) {
        int st = ptr.status, plen = 0;
        float pa = 1.f;  // lane m: scalar gate of path node m
        if (st == BOLE_TREE_OK && ptr.n > 0) {
            const int pn = ptr.n;
            const bool len_ok = plen_raw >= 0 && plen_raw <= lc.max_path;
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
            if (plen > 0 && lane < plen) pa = ly.prev_gate[(size_t)(ptr.lo + x) * H + h];
            const int row = (st == BOLE_TREE_OK && lane < plen) ? ptr.lo + x : -1;
            if (first) {
                if (lane == 0 && lc.tree_status) lc.tree_status[b] = st;
                if (lc.path_nodes && lane < lc.max_path) lc.path_nodes[(size_t)b * lc.max_path + lane] = row;
            }
        } else {
            if (st == BOLE_TREE_OK && plen_raw != 0) st = BOLE_TREE_BAD_PATH;  // empty tree
            if (first) {
                if (lane == 0 && lc.tree_status) lc.tree_status[b] = st;
                if (lc.path_nodes && lane < lc.max_path) lc.path_nodes[(size_t)b * lc.max_path + lane] = -1;
            }
        }
        if (plen > 0) {
            // stage kLazyStage path nodes at a time: chunk c of the stage is node c / LCPN
            for (int m0 = 0; m0 < plen; m0 += kLazyStage) {
                const int mc = min(kLazyStage, plen - m0);
#pragma unroll
                for (int u = 0; u < LCH; ++u) {
                    const int c = lane + 64 * u;
                    const int m = c / LCPN, part = c - m * LCPN;
                    // every lane takes part in the shuffle; only m < mc use the result
                    const int xs = __shfl(lpx, min(m0 + m, 63), 64);
                    if (m < mc) {
                        bf16x8 chunk;
                        if (m0 == 0) {
                            chunk = pf[u];  // prefetched: plen == plen_raw here
                        } else {
                            const size_t prow = (size_t)(ptr.lo + min(max(xs, 0), ptr.n - 1)) * H + h;
                            chunk = part < LCK
                                        ? load16(static_cast<const __bf16 *>(ly.prev_k) + prow * DK + 8 * part)
                                        : load16(static_cast<const __bf16 *>(ly.prev_v) + prow * DV +
                                                 c0 + 8 * (part - LCK));
                        }
                        if (part < LCK)
                            *reinterpret_cast<bf16x8 *>(s_pk + m * DK + 8 * part) = chunk;
                        else
                            *reinterpret_cast<bf16x8 *>(s_pv + m * CW + 8 * (part - LCK)) = chunk;
                    }
                }
                for (int m = 0; m < mc; ++m) {
                    const float a = readlane_f(pa, m0 + m);
                    const vvec vv = *reinterpret_cast<const vvec *>(s_pv + m * CW + CPL * n16);
#pragma unroll
                    for (int t = 0; t < KT; ++t) {
                        const bf16x8 kk = *reinterpret_cast<const bf16x8 *>(s_pk + m * DK + 32 * t + 8 * g);
#pragma unroll
                        for (int e = 0; e < 8; ++e)
#pragma unroll
                            for (int c = 0; c < CPL; ++c)
                                hreg[8 * t + e][c] = a * hreg[8 * t + e][c] +
                                                     static_cast<float>(kk[e]) * static_cast<float>(vv[c]);
                    }
                }
            }
#pragma unroll
            for (int s = 0; s < HS; ++s)
                __builtin_nontemporal_store(hreg[s], reinterpret_cast<hvec *>(
                    hu + ((uint32_t)(32 * (s >> 3) + 8 * g + (s & 7)) * DV + CPL * n16)));
        }
        if (!do_verify) return;
    }

    // ---- 2. topology and base-2 cumulative decay, lane = node (every wavefront)
    const float lg2 = lane < n ? __builtin_amdgcn_logf(g_raw) : 0.f;
    const WaveTopoL topo = wave_topology_cumlog(p_raw, lg2, n);
    if (writer) tree_status[b] = topo.bad;
    if (topo.bad) {
        for (int i = g; i < n; i += 4)
#pragma unroll
            for (int c = 0; c < CPL; ++c)
                ou[(uint32_t)i * rv + CPL * n16 + c] = __builtin_nanf("");
        return;
    }
    const float L2 = topo.L;

    // ---- 3. H_0 term: over the 8 loads of k-step t, lane (n, g) holds rows 32t + 8g + e
    // of columns CPL*n + c: the B operand for column tile c; A is the Q fragment.
    f32x4 acc[NT][CPL];
#pragma unroll
    for (int it = 0; it < NT; ++it)
#pragma unroll
        for (int c = 0; c < CPL; ++c) acc[it][c] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < KT; ++t) {
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            bf16x8 bh, bl;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                __bf16 xh, xl;
                split_bf16(hreg[8 * t + e][c], xh, xl);
                bh[e] = xh;
                bl[e] = xl;
            }
#pragma unroll
            for (int it = 0; it < NT; ++it) {
                acc[it][c] = mfma16_bf16(qf[it][t], bh, acc[it][c]);
                acc[it][c] = mfma16_bf16(qf[it][t], bl, acc[it][c]);
            }
        }
    }
    // row scale 2^{L_i}, node 16it + 4g + r
#pragma unroll
    for (int it = 0; it < NT; ++it)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float sc = __builtin_amdgcn_exp2f(__shfl(L2, 16 * it + 4 * g + r, 64));
#pragma unroll
            for (int c = 0; c < CPL; ++c) acc[it][c][r] *= sc;
        }

    // ---- 4. intra-tree term, one node tile and one ancestor tile pair at a time
#pragma unroll
    for (int it = 0; it < NT; ++it) {
        const int ti = it;                        // node tile
        const int i = 16 * ti + n16;              // node of this lane's column
        const uint64_t mi = shfl_u64(topo.mask, i);
        const float Li = __shfl(L2, i, 64);
#pragma unroll
        for (int p = 0; p < NN / 32; ++p) {       // ancestor tile pair (2p, 2p+1)
            if (2 * p > ti) break;                // wave-uniform: nothing above the diagonal
            float w[8];
#pragma unroll
            for (int hlf = 0; hlf < 2; ++hlf) {
                const int jt = 2 * p + hlf;
                f32x4 st = {0.f, 0.f, 0.f, 0.f};
                if (jt <= ti) {
#pragma unroll
                    for (int t = 0; t < KT; ++t) {
                        const int j = 16 * jt + n16, pc = 4 * t + g;
                        st = mfma16_bf16(s_k[j * PPR + (pc ^ (j % PPR))], qf[it][t], st);
                    }
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int j = 16 * jt + 4 * g + r;
                    const bool anc = jt <= ti && ((mi >> j) & 1ull);
                    const float d = __builtin_amdgcn_exp2f(Li - __shfl(L2, j, 64));
                    w[4 * hlf + r] = anc ? st[r] * d : 0.f;
                }
            }
            bf16x8 wh, wl;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                __bf16 xh, xl;
                split_bf16(w[e], xh, xl);
                wh[e] = xh;
                wl[e] = xl;
            }
            // V operand for column tile c: element e = V[32p + j(e)][CPL*n + c]
            bf16x8 vb[CPL];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int j = 32 * p + (e < 4 ? 4 * g + e : 12 + 4 * g + e);
                const vvec x = *reinterpret_cast<const vvec *>(s_v + j * CW + CPL * n16);
#pragma unroll
                for (int c = 0; c < CPL; ++c) vb[c][e] = x[c];
            }
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
                acc[it][c] = mfma16_bf16(wh, vb[c], acc[it][c]);
                acc[it][c] = mfma16_bf16(wl, vb[c], acc[it][c]);
            }
        }
    }

    // ---- 5. store: node 16it + 4g + r, columns CPL*n .. +CPL-1
#pragma unroll
    for (int it = 0; it < NT; ++it)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = 16 * it + 4 * g + r;
            hvec o;
#pragma unroll
            for (int c = 0; c < CPL; ++c) o[c] = acc[it][c][r];
            if (i < n)
                __builtin_nontemporal_store(o, reinterpret_cast<hvec *>(ou + ((uint32_t)i * rv + CPL * n16)));
        }
}

// Trees of up to 64 nodes on two wavefronts that split H_0's rows: wavefront w loads
// rows [DK/2 w, DK/2 (w+1)) of the slice (all CW columns, 16-byte loads as above) and
// forms the H_0 term of every node tile over those rows; the two halves meet in LDS,
// where each wavefront hands the other the partial sums of the other's node tiles (node
// tiles 2w, 2w+1 belong to wavefront w). H_0 is read once, with the same full-width row
// loads as the one-wavefront kernel, and each wavefront then finishes the intra-tree
// term and the store of its own node tiles. Node tiles past the tree are skipped
// (wave-uniform); K and V rows are staged per pair of tiles, clamped into the tree, so
// every V row that a masked (zero) weight meets is finite. Every other tree, and the
// status of out-of-range trees, is the one-wavefront kernel's.
template <int DK, int DV, int CWM>
constexpr int ksplit_smem_bytes() {
    return 64 * (DK / 8) * 16 + 64 * (DV < CWM ? DV : CWM) * 2;
}

// LAZY: the unit's state first takes the previous step's accepted path, with the rules and
// outputs of bole_commit_path (as in the one-wavefront lazy body), each wavefront updating
// and writing back the H_0 rows it holds; the tree is then verified against the new state.
// Path factors are staged kLazyStage path nodes at a time in `lsmem`, this wavefront's own
// kLazyStage * (DK / 2 + CW) bf16: the k elements of its rows and the v columns.
template <int DK, int DV, int CWM>
constexpr int ksplit_lazy_smem_elems() {
    return 8 * (DK / 2 + (DV < CWM ? DV : CWM));
}

// Both wavefronts of a 128-thread workgroup (or a pair of a packed one); smem holds
// ksplit_smem_bytes bytes. `known`: the tree range of the unit's sequence, else read here.
template <int DK, int DV, bool LAZY, int CWM>
__device__ __forceinline__ void ksplit_body(
    const bole_layer_t ly, const int32_t *__restrict__ parent,
    const int32_t *__restrict__ node_offsets, int32_t *__restrict__ tree_status, int H, int T,
    int U, int max_n, char *smem, int unit_g1, int w_in, const LazyCommit &lc, __bf16 *lsmem,
    const TreeRange *known) {
    constexpr int CW = DV < CWM ? DV : CWM; // state columns per workgroup
    constexpr int CPL = CW / 16;            // columns per lane: 4 or 2
    constexpr int G = DV / CW;              // column groups per unit
    constexpr int KT = DK / 32;             // k-steps of the bf16 products
    constexpr int KH = KT / 2;              // k-steps of H_0 rows per wavefront
    constexpr int HSW = 8 * KH;             // H_0 loads per lane (4 rows each per wavefront)
    constexpr int PPR = DK / 8;             // 16-byte pieces per K row
    constexpr int VPR = CW / 8;             // 16-byte pieces per V row
    constexpr int NN = 64;
    typedef float hvec __attribute__((ext_vector_type(CPL)));
    typedef __bf16 vvec __attribute__((ext_vector_type(CPL)));
    // K rows: piece p of row j at slot j*PPR + (p ^ j%PPR); then one region used twice:
    // first for the partials handed from one wavefront to the other, then for the V rows
    // of the group's columns (row j at [CW j]). Both take 128 CW bytes.
    static_assert(2 * CPL * 64 * sizeof(f32x4) == NN * CW * sizeof(__bf16), "shared region");
    bf16x8 *const s_k = reinterpret_cast<bf16x8 *>(smem);
    f32x4 *const s_x = reinterpret_cast<f32x4 *>(s_k + NN * PPR);
    __bf16 *const s_v = reinterpret_cast<__bf16 *>(s_x);
    const __bf16 *const q = static_cast<const __bf16 *>(ly.q);
    const __bf16 *const k = static_cast<const __bf16 *>(ly.k);
    const __bf16 *const v = static_cast<const __bf16 *>(ly.v);
    const float *const gate = ly.gate;
    float *const out = ly.out;

    const int lane = lane_id();
    const int w = __builtin_amdgcn_readfirstlane(w_in);  // wavefront of the unit, 0 or 1
    const int n16 = lane & 15, g = lane >> 4;
    int unit, cg;
    if (G == 1) {
        unit = unit_g1;
        if (unit >= U) return;  // uniform over the unit's two wavefronts
        cg = 0;
    } else {
        const int slot = blockIdx.x >> 3;
        cg = slot % G;
        unit = (slot / G) * 8 + (blockIdx.x & 7);
        if (unit >= U) return;
    }
    const int b = unit / H, h = unit - b * H;
    const int c0 = cg * CW;
    const bool first = blockIdx.y == 0 && h == 0 && cg == 0;
    const bool writer = tree_status != nullptr && first && w == 0 && lane_id() == 0;

    const TreeRange tr = known ? *known : tree_range(node_offsets, b, T, max_n);
    if (tr.status != BOLE_TREE_OK || tr.n <= 32) return;
    const int n = tr.n;
    const int lo = tr.lo, last = n - 1;
    const int ntl = (n + 15) >> 4;          // node tiles holding nodes
    const int rows = n > 32 ? 64 : 32;      // K and V rows staged (whole tile pairs)
    const uint32_t rq = (uint32_t)H * DK, rv = (uint32_t)H * DV;
    const __bf16 *qu = q + (size_t)lo * rq + (size_t)h * DK;
    const __bf16 *ku = k + (size_t)lo * rq + (size_t)h * DK;
    const __bf16 *vu = v + (size_t)lo * rv + (size_t)h * DV + c0;
    float *ou = out + (size_t)lo * rv + (size_t)h * DV + c0;
    float *hu = ly.H0 + (size_t)unit * DK * DV + c0;  // written only by the lazy commit

    // lazy commit, first: the previous tree's offsets, its parent links and the path
    // indices (lane m: path position m; lx: the path node of each factor chunk this lane
    // stages first). A chunk is 16 bytes of a path node's k elements on this wavefront's
    // rows, or of its v row's group columns.
    constexpr int kStage = 8;               // path nodes staged at a time
    constexpr int DKH = DK / 2;             // k elements of this wavefront's rows
    constexpr int LCK = DKH / 8, LCV = CW / 8, LCPN = LCK + LCV;
    constexpr int LCH = LAZY ? (kStage * LCPN + 63) / 64 : 1;
    static_assert(!LAZY || ksplit_lazy_smem_elems<DK, DV, CWM>() == kStage * (DKH + CW), "staging");
    TreeRange ptr = {0, 0, BOLE_TREE_OK};
    int plen_raw = 0;
    bool plikely = false;
    int lx[LCH];
    int lpx = -1, lpp = -1;
    if constexpr (LAZY) {
        ptr = tree_range(lc.node_offsets, b, lc.T, lc.max_n);
        plen_raw = lc.accepted_len[b];
        plikely = ptr.status == BOLE_TREE_OK && plen_raw > 0 && plen_raw <= lc.max_path &&
                  plen_raw <= ptr.n;
        const int32_t *acc_b = lc.accepted_idx + (size_t)b * lc.max_path;
#pragma unroll
        for (int u = 0; u < LCH; ++u) {
            const int m = (lane + 64 * u) / LCPN;
            lx[u] = (plikely && m < plen_raw) ? acc_b[m] : 0;
        }
        if (ptr.status == BOLE_TREE_OK && ptr.n > 0) {
            lpp = lane < ptr.n ? lc.parent[ptr.lo + lane] : -1;
            if (lane < plen_raw && plen_raw <= lc.max_path) lpx = acc_b[lane];
        }
    }

    // ---- 1. issue every load. Relative node tile r: r < 2 is own tile 2w + r, r >= 2
    // the other wavefront's tile 2(1 - w) + r - 2.
    const uint32_t node = (uint32_t)min(lane, last);
    const int p_raw = parent[lo + node];
    const float g_raw = gate[(size_t)lo * H + h + node * (uint32_t)H];
    // qa[r][tl]: Q fragment of relative tile r at this wavefront's k-step w*KH + tl;
    // qb[r][tl] (loaded after the H_0 term, which does not need it): own tile r at the
    // other wavefront's k-step (1 - w)*KH + tl. The other wavefront's tiles (r >= 2) are
    // read again there, as its qb: they take plain loads, which leave the lines in L2 for
    // that second read (streaming loads did not, and it went to HBM: 64-node trees 74.0
    // -> 65.2 us, the ragged batch 51.4 -> 47.2 us)
    bf16x8 qa[4][KH], qb[2][KH];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int ti = r < 2 ? 2 * w + r : 2 * (1 - w) + r - 2;
        const __bf16 *qrow = qu + (uint32_t)min(16 * ti + n16, last) * rq + 8 * g;
#pragma unroll
        for (int tl = 0; tl < KH; ++tl) {
            qa[r][tl] = bf16x8{};
            if (ti < ntl)
                qa[r][tl] = (r >= 2 || G > 1) ? load16(qrow + 32 * (w * KH + tl))
                                              : load16_stream(qrow + 32 * (w * KH + tl));
        }
    }
    // K: load s = w + 2u fills LDS slots 64s .. 64s+63 (rows (64/PPR)s ..); V: load s,
    // rows (64/VPR)s + lane/VPR. Only rows below `rows` are staged.
    constexpr int KL = NN * PPR / 128, VL = NN * VPR / 128;
    bf16x8 kst[KL], vst[VL];
#pragma unroll
    for (int u = 0; u < KL; ++u) {
        const int s = w + 2 * u;
        const int j = (64 / PPR) * s + lane / PPR;
        const int pc = (lane % PPR) ^ (j % PPR);
        // (G > 1: every column group's workgroup reads these rows, as the q rows)
        if ((64 / PPR) * s < rows)
            kst[u] = G > 1 ? load16(ku + ((uint32_t)min(j, last) * rq + 8 * pc))
                           : load16_stream(ku + ((uint32_t)min(j, last) * rq + 8 * pc));
    }
    // H_0 rows of this wavefront: load s = 8tl + e, lane (n, g): row 32(w*KH + tl) + 8g + e
    hvec hreg[HSW];
#pragma unroll
    for (int s = 0; s < HSW; ++s)
        hreg[s] = __builtin_nontemporal_load(reinterpret_cast<const hvec *>(
            hu + ((uint32_t)(32 * (w * KH + (s >> 3)) + 8 * g + (s & 7)) * DV + CPL * n16)));
    // lazy commit: the factor chunks of the first kStage path nodes, issued behind H_0 and
    // held in registers until the path is validated; rows clamped into the previous tree,
    // which its offsets check keeps inside [0, T)
    bf16x8 pf[LCH];
    if constexpr (LAZY) {
        if (plikely) {
            const int mc0 = min(kStage, plen_raw);
#pragma unroll
            for (int u = 0; u < LCH; ++u) {
                const int c = lane + 64 * u;
                const int m = c / LCPN, part = c - m * LCPN;
                if (m < mc0) {
                    const size_t prow = (size_t)(ptr.lo + min(max(lx[u], 0), ptr.n - 1)) * H + h;
                    pf[u] = part < LCK
                                ? load16(static_cast<const __bf16 *>(ly.prev_k) + prow * DK +
                                         w * DKH + 8 * part)
                                : load16(static_cast<const __bf16 *>(ly.prev_v) + prow * DV + c0 +
                                         8 * (part - LCK));
                }
            }
        }
    }
#pragma unroll
    for (int u = 0; u < KL; ++u)
        if ((64 / PPR) * (w + 2 * u) < rows) s_k[64 * (w + 2 * u) + lane] = kst[u];

    // ---- lazy commit: validate the previous path, stage its factors, update this
    // wavefront's H_0 rows in registers and write them back (both wavefronts validate;
    // the first writes the per-tree outputs)
    if constexpr (LAZY) {
        const bool lfirst = first && w == 0;
        int st = ptr.status, plen = 0;
        float pa = 1.f;  // lane m: scalar gate of path node m
        if (st == BOLE_TREE_OK && ptr.n > 0) {
            const int pn = ptr.n;
            const bool len_ok = plen_raw >= 0 && plen_raw <= lc.max_path;
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
            if (plen > 0 && lane < plen) pa = ly.prev_gate[(size_t)(ptr.lo + x) * H + h];
            const int row = (st == BOLE_TREE_OK && lane < plen) ? ptr.lo + x : -1;
            if (lfirst) {
                if (lane == 0 && lc.tree_status) lc.tree_status[b] = st;
                if (lc.path_nodes && lane < lc.max_path) lc.path_nodes[(size_t)b * lc.max_path + lane] = row;
            }
        } else {
            if (st == BOLE_TREE_OK && plen_raw != 0) st = BOLE_TREE_BAD_PATH;  // empty tree
            if (lfirst) {
                if (lane == 0 && lc.tree_status) lc.tree_status[b] = st;
                if (lc.path_nodes && lane < lc.max_path) lc.path_nodes[(size_t)b * lc.max_path + lane] = -1;
            }
        }
        if (plen > 0) {
            __bf16 *const s_pk = lsmem, *const s_pv = lsmem + kStage * DKH;
            for (int m0 = 0; m0 < plen; m0 += kStage) {
                const int mc = min(kStage, plen - m0);
#pragma unroll
                for (int u = 0; u < LCH; ++u) {
                    const int c = lane + 64 * u;
                    const int m = c / LCPN, part = c - m * LCPN;
                    // every lane takes part in the shuffle; only m < mc use the result
                    const int xs = __shfl(lpx, min(m0 + m, 63), 64);
                    if (m < mc) {
                        bf16x8 chunk;
                        if (m0 == 0) {
                            chunk = pf[u];  // prefetched: plen == plen_raw here
                        } else {
                            const size_t prow = (size_t)(ptr.lo + min(max(xs, 0), ptr.n - 1)) * H + h;
                            chunk = part < LCK
                                        ? load16(static_cast<const __bf16 *>(ly.prev_k) + prow * DK +
                                                 w * DKH + 8 * part)
                                        : load16(static_cast<const __bf16 *>(ly.prev_v) + prow * DV +
                                                 c0 + 8 * (part - LCK));
                        }
                        if (part < LCK)
                            *reinterpret_cast<bf16x8 *>(s_pk + m * DKH + 8 * part) = chunk;
                        else
                            *reinterpret_cast<bf16x8 *>(s_pv + m * CW + 8 * (part - LCK)) = chunk;
                    }
                }
                for (int m = 0; m < mc; ++m) {
                    const float a = readlane_f(pa, m0 + m);
                    const vvec vv = *reinterpret_cast<const vvec *>(s_pv + m * CW + CPL * n16);
#pragma unroll
                    for (int tl = 0; tl < KH; ++tl) {
                        const bf16x8 kk = *reinterpret_cast<const bf16x8 *>(s_pk + m * DKH + 32 * tl + 8 * g);
#pragma unroll
                        for (int e = 0; e < 8; ++e)
#pragma unroll
                            for (int c = 0; c < CPL; ++c)
                                hreg[8 * tl + e][c] = a * hreg[8 * tl + e][c] +
                                                      static_cast<float>(kk[e]) * static_cast<float>(vv[c]);
                    }
                }
            }
#pragma unroll
            for (int s = 0; s < HSW; ++s)
                __builtin_nontemporal_store(hreg[s], reinterpret_cast<hvec *>(
                    hu + ((uint32_t)(32 * (w * KH + (s >> 3)) + 8 * g + (s & 7)) * DV + CPL * n16)));
        }
    }

    // ---- 2. topology and base-2 cumulative decay (both wavefronts, same result)
    const float lg2 = lane < n ? __builtin_amdgcn_logf(g_raw) : 0.f;
    const WaveTopoL topo = wave_topology_cumlog(p_raw, lg2, n);
    if (writer) tree_status[b] = topo.bad;
    if (topo.bad) {
        for (int i = g + 4 * w; i < n; i += 8)
#pragma unroll
            for (int c = 0; c < CPL; ++c) ou[(uint32_t)i * rv + CPL * n16 + c] = __builtin_nanf("");
        return;
    }
    const float L2 = topo.L;

    // ---- 3. H_0 term over this wavefront's rows, for every node tile in the tree
    f32x4 acc[4][CPL];
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int c = 0; c < CPL; ++c) acc[r][c] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int tl = 0; tl < KH; ++tl) {
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            bf16x8 bh, bl;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                __bf16 xh, xl;
                split_bf16(hreg[8 * tl + e][c], xh, xl);
                bh[e] = xh;
                bl[e] = xl;
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int ti = r < 2 ? 2 * w + r : 2 * (1 - w) + r - 2;
                if (ti < ntl) {
                    acc[r][c] = mfma16_bf16(qa[r][tl], bh, acc[r][c]);
                    acc[r][c] = mfma16_bf16(qa[r][tl], bl, acc[r][c]);
                }
            }
        }
    }
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const int ti = 2 * w + r;
        const __bf16 *qrow = qu + (uint32_t)min(16 * ti + n16, last) * rq + 8 * g;
#pragma unroll
        for (int tl = 0; tl < KH; ++tl) {
            qb[r][tl] = bf16x8{};
            if (ti < ntl)
                qb[r][tl] = G > 1 ? load16(qrow + 32 * ((1 - w) * KH + tl))
                                  : load16_stream(qrow + 32 * ((1 - w) * KH + tl));
        }
    }
    // V rows, needed only by the intra-tree term and staged after the swap in the region
    // the partials use: issued here, once H_0's registers are free
#pragma unroll
    for (int u = 0; u < VL; ++u) {
        const int s = w + 2 * u;
        const int j = (64 / VPR) * s + lane / VPR;
        if ((64 / VPR) * s < rows)
            vst[u] = load16_stream(vu + ((uint32_t)min(j, last) * rv + 8 * (lane % VPR)));
    }
    // hand the other wavefront its partials (same accumulator layout in both) and take
    // ours, through one region in two phases: wavefront 1 hands over tiles 0 and 1, then
    // wavefront 0 tiles 2 and 3
#pragma unroll
    for (int ph = 0; ph < 2; ++ph) {
        const int src = 1 - ph;               // the wavefront writing in this phase
        if (w == src)
#pragma unroll
            for (int r = 0; r < 2; ++r)
                if (2 * ph + r < ntl)
#pragma unroll
                    for (int c = 0; c < CPL; ++c) s_x[(r * CPL + c) * 64 + lane] = acc[2 + r][c];
        __syncthreads();  // (the first also publishes both halves of K)
        if (w != src)
#pragma unroll
            for (int r = 0; r < 2; ++r)
                if (2 * ph + r < ntl)
#pragma unroll
                    for (int c = 0; c < CPL; ++c) acc[r][c] += s_x[(r * CPL + c) * 64 + lane];
        __syncthreads();  // read before the second phase, then V, overwrite the region
    }
#pragma unroll
    for (int u = 0; u < VL; ++u)
        if ((64 / VPR) * (w + 2 * u) < rows)
            *reinterpret_cast<bf16x8 *>(s_v + 512 * (w + 2 * u) + 8 * lane) = vst[u];
    __syncthreads();
    if (2 * w >= ntl) return;  // no node tile of this wavefront's in the tree
    // row scale 2^{L_i}, node 16ti + 4g + rr
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const float sc = __builtin_amdgcn_exp2f(__shfl(L2, 16 * (2 * w + r) + 4 * g + rr, 64));
#pragma unroll
            for (int c = 0; c < CPL; ++c) acc[r][c][rr] *= sc;
        }

    // ---- 4. intra-tree term for own node tiles, one ancestor tile pair at a time
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const int ti = 2 * w + r;               // node tile (wave-uniform)
        if (ti >= ntl) break;
        const int i = 16 * ti + n16;            // node of this lane's column
        const uint64_t mi = shfl_u64(topo.mask, i);
        const float Li = __shfl(L2, i, 64);
#pragma unroll
        for (int p = 0; p < 2; ++p) {           // ancestor tile pair (2p, 2p+1)
            if (2 * p > ti) break;
            float wv[8];
#pragma unroll
            for (int hlf = 0; hlf < 2; ++hlf) {
                const int jt = 2 * p + hlf;
                f32x4 st = {0.f, 0.f, 0.f, 0.f};
                if (jt <= ti) {
#pragma unroll
                    for (int t = 0; t < KT; ++t) {
                        const int j = 16 * jt + n16, pc = 4 * t + g;
                        const bf16x8 qq = (t / KH == w) ? qa[r][t % KH] : qb[r][t % KH];
                        st = mfma16_bf16(s_k[j * PPR + (pc ^ (j % PPR))], qq, st);
                    }
                }
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    const int j = 16 * jt + 4 * g + rr;
                    const bool anc = jt <= ti && ((mi >> j) & 1ull);
                    const float d = __builtin_amdgcn_exp2f(Li - __shfl(L2, j, 64));
                    wv[4 * hlf + rr] = anc ? st[rr] * d : 0.f;
                }
            }
            bf16x8 wh, wl;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                __bf16 xh, xl;
                split_bf16(wv[e], xh, xl);
                wh[e] = xh;
                wl[e] = xl;
            }
            bf16x8 vb[CPL];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int j = 32 * p + (e < 4 ? 4 * g + e : 12 + 4 * g + e);
                const vvec x = *reinterpret_cast<const vvec *>(s_v + j * CW + CPL * n16);
#pragma unroll
                for (int c = 0; c < CPL; ++c) vb[c][e] = x[c];
            }
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
                acc[r][c] = mfma16_bf16(wh, vb[c], acc[r][c]);
                acc[r][c] = mfma16_bf16(wl, vb[c], acc[r][c]);
            }
        }
    }

    // ---- 5. store own node tiles: node 16ti + 4g + rr, columns CPL*n ..
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const int i = 16 * (2 * w + r) + 4 * g + rr;
            hvec o;
#pragma unroll
            for (int c = 0; c < CPL; ++c) o[c] = acc[r][c][rr];
            if (i < n)
                __builtin_nontemporal_store(o, reinterpret_cast<hvec *>(ou + ((uint32_t)i * rv + CPL * n16)));
        }
}

static bool shape_ok(const bole_dims_t &d) {
    if (d.flags & BOLE_FLAG_FORCE_GENERIC) return false;
    if (d.factor_dtype != BOLE_DTYPE_BF16 || d.gate_kind != BOLE_GATE_SCALAR) return false;
    if (d.d_k != 64 && d.d_k != 128) return false;
    if (d.d_v != 32 && d.d_v != 64 && d.d_v != 128 && d.d_v != 256) return false;
    // per-tree element offsets (64 rows of one head's rows, and one H_0 slice) are 32-bit
    const uint64_t row_elems = (uint64_t)d.heads * (uint64_t)(d.d_k > d.d_v ? d.d_k : d.d_v);
    if (row_elems * kMaxTree >= (1ull << 31)) return false;
    // work slots (unit x column group, padded to 8) fit an int
    const uint64_t groups = d.d_v > 64 ? (uint64_t)d.d_v / 64 : 1;
    return ((uint64_t)d.batch * (uint64_t)d.heads + 8) * groups < (1ull << 30);
}

bool verify_mfma_applies(const bole_dims_t &d, const bole_layer_t *layers, int nl) {
    if (!shape_ok(d)) return false;
    // 16-byte loads of H_0, q, k, v rows and 16-byte stores of out rows
    for (int l = 0; l < nl; ++l) {
        const bole_layer_t &y = layers[l];
        const uintptr_t a = reinterpret_cast<uintptr_t>(y.H0) | reinterpret_cast<uintptr_t>(y.q) |
                            reinterpret_cast<uintptr_t>(y.k) | reinterpret_cast<uintptr_t>(y.v) |
                            reinterpret_cast<uintptr_t>(y.out);
        if (a % 16 != 0) return false;
    }
    return true;
}

// Units (sequence x head x layer) from which the one-wavefront kernels take several units
// per workgroup (kVerifyGroup for verify, kLazyGroup for the lazy commit, measured best):
// below it, one unit per workgroup keeps more CUs busy.
constexpr uint64_t kGroupMinUnits = 2048;
constexpr int kVerifyGroup = 2;
constexpr int kLazyGroup = 4;
// Sequences up to which the fused launch is packed (every wavefront reads all tree offsets),
// and its wavefront slots per workgroup (eight, one workgroup per CU, measured slower)
constexpr int kPackMaxSeq = 1024;
constexpr int kPackSlots = 4;
// Launches of at most this many units (sequence x head x layer) at d_v = 64 take two
// 32-column groups per unit: twice the workgroups, each with half the H_0 slice and half
// the products, for batches too small to fill the chip (the groups of a unit share its q
// and k rows through L2). Measured (cold): 256 units of 32-node trees 6.4 -> 5.9 us, their
// lazy step 10.4 -> 9.8 us, 128 units of 64-node trees 7.7 -> 6.7 us, 256 of them
// unchanged. At 512 units, 32-node trees gain (8.4 -> 8.0 us) but 64-node trees lose
// (12.3 -> 12.5-13.3 us), so the larger limit holds only under the 32-node budget; at 1,024
// units both lose.
constexpr uint64_t kHalfColumnsMaxUnits = 256;
constexpr uint64_t kHalfColumnsMaxUnitsBudget32 = 512;

template <int DK, int DV, int CWM>
static void launch_shape_cw(const bole_layer_t *layers, int nl, const int32_t *parent,
                            const int32_t *node_offsets, const bole_dims_t &d,
                            int32_t *tree_status, hipStream_t stream, const LazyCommit *lazy) {
    const unsigned U = (unsigned)d.batch * (unsigned)d.heads;
    const int max_n = max_tree_nodes(d.flags);
    // one workgroup per (unit, column group, layer): G > 1: ceil(U / 8) slots of 8 units,
    // each slot G column groups wide, so the groups of a unit share an XCD
    constexpr int G = DV < CWM ? 1 : DV / CWM;
    const dim3 grid(G == 1 ? U : ((U + 7) / 8) * 8 * G, (unsigned)nl);
    // groups of units once the launch holds enough of them; a small batch keeps one unit per
    // workgroup, so that more CUs take part
    const bool group = G == 1 && (uint64_t)U * (uint64_t)nl >= kGroupMinUnits;
    constexpr int NV = G == 1 ? kVerifyGroup : 1, NL = G == 1 ? kLazyGroup : 1;
    const dim3 vgrid((U + NV - 1) / NV, (unsigned)nl), lgrid((U + NL - 1) / NL, (unsigned)nl);
    LayerTable lt = {};
    for (int l = 0; l < nl; ++l) lt.l[l] = layers[l];
    const LazyCommit none = {};
    const int H = d.heads, T = d.total_nodes;
    // the packed fused launch: slots for every unit taking two, so half a workgroup per unit
    const bool pack = group && G == 1 && H % kPackSlots == 0 && d.batch <= kPackMaxSeq;
    const dim3 pgrid(2 * U / kPackSlots, (unsigned)nl), pblock(64 * kPackSlots);
    if (lazy && max_n > 32) {
        // every tree size in one launch, as the fused verify below, each body committing
        // the units whose trees it verifies
        if (pack)
            verify_mfma_tree_kernel<DK, DV, true, true, G == 1 ? kPackSlots : 1, CWM><<<pgrid, pblock, 0, stream>>>(
                lt, parent, node_offsets, tree_status, H, T, (int)U, max_n, *lazy);
        else if (group && H % 2 == 0)
            verify_mfma_tree_kernel<DK, DV, true, true, G == 1 ? 2 : 1, CWM><<<
                dim3(G == 1 ? (U + 1) / 2 : grid.x, (unsigned)nl), dim3(G == 1 ? 256 : 128), 0, stream>>>(
                lt, parent, node_offsets, tree_status, H, T, (int)U, max_n, *lazy);
        else
            verify_mfma_tree_kernel<DK, DV, true, true, 1, CWM><<<grid, dim3(128), 0, stream>>>(
                lt, parent, node_offsets, tree_status, H, T, (int)U, max_n, *lazy);
    } else if (lazy) {
        if (group)
            verify_mfma_tree_kernel<DK, DV, true, false, NL, CWM><<<lgrid, dim3(64 * NL), 0, stream>>>(
                lt, parent, node_offsets, tree_status, H, T, (int)U, max_n, *lazy);
        else
            verify_mfma_tree_kernel<DK, DV, true, false, 1, CWM><<<grid, dim3(64), 0, stream>>>(
                lt, parent, node_offsets, tree_status, H, T, (int)U, max_n, *lazy);
    } else if (max_n > 32) {
        // two units per workgroup only when they always share a tree (an even head count)
        if (pack)
            verify_mfma_tree_kernel<DK, DV, false, true, G == 1 ? kPackSlots : 1, CWM><<<pgrid, pblock, 0, stream>>>(
                lt, parent, node_offsets, tree_status, H, T, (int)U, max_n, none);
        else if (group && H % 2 == 0)
            verify_mfma_tree_kernel<DK, DV, false, true, G == 1 ? 2 : 1, CWM><<<
                dim3(G == 1 ? (U + 1) / 2 : grid.x, (unsigned)nl), dim3(G == 1 ? 256 : 128), 0, stream>>>(
                lt, parent, node_offsets, tree_status, H, T, (int)U, max_n, none);
        else
            verify_mfma_tree_kernel<DK, DV, false, true, 1, CWM><<<grid, dim3(128), 0, stream>>>(
                lt, parent, node_offsets, tree_status, H, T, (int)U, max_n, none);
    } else if (group) {
        verify_mfma_tree_kernel<DK, DV, false, false, NV, CWM><<<vgrid, dim3(64 * NV), 0, stream>>>(
            lt, parent, node_offsets, tree_status, H, T, (int)U, max_n, none);
    } else {
        verify_mfma_tree_kernel<DK, DV, false, false, 1, CWM><<<grid, dim3(64), 0, stream>>>(
            lt, parent, node_offsets, tree_status, H, T, (int)U, max_n, none);
    }
}

template <int DK, int DV>
static void launch_shape(const bole_layer_t *layers, int nl, const int32_t *parent,
                         const int32_t *node_offsets, const bole_dims_t &d, int32_t *tree_status,
                         hipStream_t stream, const LazyCommit *lazy) {
    if constexpr (DV == 64) {
        const uint64_t units = (uint64_t)d.batch * (uint64_t)d.heads * (uint64_t)nl;
        const uint64_t limit = max_tree_nodes(d.flags) <= 32 ? kHalfColumnsMaxUnitsBudget32
                                                              : kHalfColumnsMaxUnits;
        if (units <= limit) {
            launch_shape_cw<DK, DV, 32>(layers, nl, parent, node_offsets, d, tree_status, stream, lazy);
            return;
        }
    }
    launch_shape_cw<DK, DV, 64>(layers, nl, parent, node_offsets, d, tree_status, stream, lazy);
}

template <int DK>
static void launch_dk(const bole_layer_t *layers, int nl, const int32_t *parent,
                      const int32_t *node_offsets, const bole_dims_t &d, int32_t *tree_status,
                      hipStream_t stream, const LazyCommit *lazy) {
    switch (d.d_v) {
        case 32: launch_shape<DK, 32>(layers, nl, parent, node_offsets, d, tree_status, stream, lazy); break;
        case 64: launch_shape<DK, 64>(layers, nl, parent, node_offsets, d, tree_status, stream, lazy); break;
        case 128: launch_shape<DK, 128>(layers, nl, parent, node_offsets, d, tree_status, stream, lazy); break;
        case 256: launch_shape<DK, 256>(layers, nl, parent, node_offsets, d, tree_status, stream, lazy); break;
        default: break;
    }
}

hipError_t launch_verify_mfma(const bole_layer_t *layers, int nl, const int32_t *parent,
                              const int32_t *node_offsets, const bole_dims_t &d,
                              int32_t *tree_status, hipStream_t stream) {
    if (d.d_k == 64)
        launch_dk<64>(layers, nl, parent, node_offsets, d, tree_status, stream, nullptr);
    else
        launch_dk<128>(layers, nl, parent, node_offsets, d, tree_status, stream, nullptr);
    return hipGetLastError();
}

bool verify_lazy_applies(const bole_dims_t &d, const bole_dims_t &pd, const bole_layer_t *layers,
                         int nl) {
    if (!verify_mfma_applies(d, layers, nl)) return false;
    // the previous step's factors: same layout and shapes, 16-byte rows
    if (pd.factor_dtype != d.factor_dtype || pd.gate_kind != d.gate_kind || pd.d_k != d.d_k ||
        pd.d_v != d.d_v || pd.heads != d.heads || pd.batch != d.batch)
        return false;
    for (int l = 0; l < nl; ++l) {
        const uintptr_t a = reinterpret_cast<uintptr_t>(layers[l].prev_k) |
                            reinterpret_cast<uintptr_t>(layers[l].prev_v);
        if (a % 16 != 0) return false;
    }
    return true;
}

hipError_t launch_verify_lazy_commit(const bole_layer_t *layers, int nl, const PrevPath &prev,
                                     const bole_dims_t &pd, const int32_t *parent,
                                     const int32_t *node_offsets, const bole_dims_t &d,
                                     int32_t *tree_status, hipStream_t stream) {
    LazyCommit lz;
    lz.parent = prev.parent;
    lz.node_offsets = prev.node_offsets;
    lz.accepted_idx = prev.accepted_idx;
    lz.accepted_len = prev.accepted_len;
    lz.path_nodes = prev.path_nodes;
    lz.tree_status = prev.tree_status;
    lz.T = pd.total_nodes;
    lz.max_path = pd.max_path;
    lz.max_n = max_tree_nodes(pd.flags);
    if (d.d_k == 64)
        launch_dk<64>(layers, nl, parent, node_offsets, d, tree_status, stream, &lz);
    else
        launch_dk<128>(layers, nl, parent, node_offsets, d, tree_status, stream, &lz);
    return hipGetLastError();
}

}  // namespace bole
