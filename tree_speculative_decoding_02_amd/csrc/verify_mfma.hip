// verify_mfma.hip - matrix-core tree verification for bf16 factors and scalar gates
// (the Mamba-2 layout).
//
// It evaluates the closed form of the Bole summary page, section 1 ("Tree-Structured
// Closed Form"), for every node of a tree at once:
//     O = diag(2^{L}) (Q H_0) + W V,   W_ij = (q_i . k_j) 2^{L_i - L_j} [j on path(i)]
// L_i is the root-first sum of log2 a over path(i). Only per-node factors are read
// (section 2, "Token-Level Factor Encoding"); no per-node state exists anywhere.
//
// Two kernels, one launch each (the second only when the batch may hold a tree of more
// than 32 nodes):
//  - verify_mfma_tree32_kernel: trees of 1..32 nodes, one wavefront per (sequence,
//    head, 64-column group), 16x16x32 bf16 products. H_0 goes from HBM straight into
//    MFMA operand registers with row-contiguous 16-byte loads, so a wavefront needs only
//    12 KB of LDS (K and V) and eight of them fit on a CU: the whole benchmark batch is
//    in flight at once.
//  - verify_mfma_big_kernel: trees of 33..64 nodes, two 32-row tiles per wavefront,
//    32x32x16 bf16 products, the H_0 slice staged in LDS.
// Both split fp32 operands (H_0, W) into bf16 hi + lo (two products, about 16 mantissa
// bits) and mask non-ancestors by select, never by multiplication, so pairs whose decay
// factor overflows can never produce NaN. Topology and the base-2 cumulative decay are
// rebuilt by each wavefront on its own 64 lanes (lane = node), with no barrier.
#include "bole_device.h"
#include "launch.h"
#include "mfma_util.h"

namespace bole {

// Trees of 33..64 nodes: two 32-row tiles. One wavefront per (sequence, head,
// 32-column slice), one workgroup per (sequence, head, 64-column group); the groups of
// one unit stay on one XCD. Per row tile:
//  1. issue Q and K fragments (16-byte loads into MFMA operand registers) and V rows
//     (DMA into LDS); on the first tile also the whole H_0 slice (DMA into LDS);
//  2. topology and base-2 cumulative decay (first tile only), while the loads fly;
//  3. H_0 term from the resident slice, then the row scale;
//  4. intra-tree term for the tile's own ancestors (V from LDS) and, on the second
//     tile, for ancestors in the first tile (direct loads);
//  5. store.
// Every tree of another size is left to verify_mfma_tree32_kernel below.
template <int DK, int DV>
__global__ __launch_bounds__((DV < 64 ? DV : 64) / 32 * 64, 2) void verify_mfma_big_kernel(
    const float *__restrict__ H0, const __bf16 *__restrict__ q, const __bf16 *__restrict__ k,
    const __bf16 *__restrict__ v, const float *__restrict__ gate,
    const int32_t *__restrict__ parent, const int32_t *__restrict__ node_offsets,
    float *__restrict__ out, int32_t *__restrict__ tree_status, int H, int T, int U) {
    constexpr int KS = DK / 16;                    // K-steps of Q.H0 and K.Q^T
    constexpr int NCH = DK / 32;                   // 32-row H_0 chunks (two K-steps each)
    constexpr int NW = (DV < 64 ? DV : 64) / 32;   // waves per workgroup
    constexpr int G = DV / (32 * NW);              // column groups per unit
    __shared__ float s_h0[NW][NCH][32 * 32];       // per wave: its whole H_0 slice, by 32-row chunk
    __shared__ __bf16 s_v[NW][32 * 32];            // per wave: V rows of the tile, row j at [32 j]

    const int lane = lane_id();
    const int wave = threadIdx.x >> 6;
    const int col = lane & 31, half = lane >> 5;
    int unit, cg;
    if (G == 1) {
        unit = blockIdx.x;
        cg = 0;
    } else {
        const int slot = blockIdx.x >> 3;
        cg = slot % G;
        unit = (slot / G) * 8 + (blockIdx.x & 7);
        if (unit >= U) return;
    }
    const int b = unit / H, h = unit - b * H;
    // wave-uniform column base (readfirstlane tells the compiler it is uniform, so the
    // base pointers below live in scalar registers)
    const int c0 = __builtin_amdgcn_readfirstlane((cg * NW + wave) * 32);
    const bool writer = tree_status != nullptr && h == 0 && cg == 0 && threadIdx.x == 0;

    // trees of 33..64 nodes only: everything else, status included, is the streaming
    // kernel's
    const TreeRange tr = tree_range(node_offsets, b, T, kMaxTree);
    if (tr.status != BOLE_TREE_OK || tr.n <= 32) return;
    const int lo = tr.lo, n = tr.n;
    const int last = n - 1;
    // Every access below is a wave-uniform base plus a 32-bit per-lane element offset
    // (the host guarantees the offsets fit), so addresses cost one register each.
    const uint32_t rq = (uint32_t)H * DK, rv = (uint32_t)H * DV;
    const __bf16 *qu = q + (size_t)lo * rq + (size_t)h * DK;
    const __bf16 *ku = k + (size_t)lo * rq + (size_t)h * DK;
    const __bf16 *vu = v + (size_t)lo * rv + (size_t)h * DV + c0;
    float *ou = out + (size_t)lo * rv + (size_t)h * DV + c0;
    const float *hu = H0 + (size_t)unit * DK * DV + c0;

    __bf16 *lv = s_v[wave];
    // H_0 chunk c (rows 32c .. 32c+31 of the slice): instruction s moves rows 32c + 8s ..
    // +7; lane l takes row 32c + 8s + l/8, columns 4(l%8) .. +3
    const uint32_t hoff = (uint32_t)(lane >> 3) * DV + 4 * (lane & 7);
    auto dma_chunk = [&](int c, float *dst) {
#pragma unroll
        for (int s = 0; s < 4; ++s) dma16(hu + (hoff + (uint32_t)(32 * c + 8 * s) * DV), dst + 256 * s);
    };
    const uint32_t qoff_half = 8 * half;
    const uint32_t ooff = col;

    // per-node scalars first, so topology can start as soon as they land
    const int p_raw = parent[lo + min(lane, last)];
    const float g_raw = gate[(size_t)lo * H + h + (uint32_t)min(lane, last) * (uint32_t)H];

    WaveTopoL topo;
    for (int it = 0; it < 2; ++it) {
        // ---- 1. issue everything this tile needs at once: Q and K fragments (registers),
        // V rows and the whole H_0 slice (DMA into LDS). Nothing later waits on a load
        // that depends on another load.
        bf16x8 qf[KS], kf[KS];
        {
            const uint32_t qo = (uint32_t)min(32 * it + col, last) * rq + qoff_half;
#pragma unroll
            for (int t = 0; t < KS; ++t) {
                qf[t] = load16(qu + (qo + 16 * t));
                kf[t] = load16(ku + (qo + 16 * t));
            }
        }
        {
            // V rows 32it .. 32it+31: instruction s moves 16 rows, lane l takes row
            // 32it + 16s + l/4, columns 8(l%4) .. +7 of the slice
#pragma unroll
            for (int s = 0; s < 2; ++s)
                dma16(vu + ((uint32_t)min(32 * it + 16 * s + (lane >> 2), last) * rv + 8 * (lane & 3)), lv + 512 * s);
        }
        if (it == 0) {
#pragma unroll
            for (int c = 0; c < NCH; ++c) dma_chunk(c, s_h0[wave][c]);
        }

        // ---- 2. topology and decay, once, while the loads fly
        if (it == 0) {
            const float lg2 = lane < n ? __builtin_amdgcn_logf(g_raw) : 0.f;
            topo = wave_topology_cumlog(p_raw, lg2, n);
            if (writer) tree_status[b] = topo.bad;
            if (topo.bad) {
                wait_all_memory();  // no DMA may still target this workgroup's LDS after exit
                for (int i = half; i < n; i += 2) ou[(uint32_t)i * rv + ooff] = __builtin_nanf("");
                return;
            }
        }
        const float L2 = topo.L;  // log2 of the path's decay product, lane = node
        // Row r of accumulator element e is 32it + 8(e/4) + 4half + e%4: the same for every
        // lane of a half, so per-row values come from uniform lane reads.
        auto row_val = [&](float x, int base, int e) {
            const int r0 = base + 8 * (e >> 2) + (e & 3);
            const float v0 = readlane_f(x, r0);
            const float v1 = readlane_f(x, r0 + 4);
            return half ? v1 : v0;
        };

        // ---- 3. H0 term over the resident slice: acc = Q_it . H0 slice, H0 split into
        // bf16 hi + lo
        f32x16 acc;
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[e] = 0.f;
        wait_all_memory();
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            const float *buf = s_h0[wave][c];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                bf16x8 bh, bl;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    __bf16 xh, xl;
                    split_bf16(buf[(16 * t + 8 * half + e) * 32 + col], xh, xl);
                    bh[e] = xh;
                    bl[e] = xl;
                }
                acc = mfma32(qf[2 * c + t], bh, acc);
                acc = mfma32(qf[2 * c + t], bl, acc);
            }
        }
        // row scale 2^{L2_i}
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[e] *= __builtin_amdgcn_exp2f(row_val(L2, 32 * it, e));

        // ---- 4. intra-tree term: ancestor tile jt = it (V from LDS), then jt = 0 for a
        // second row tile (direct loads)
        const int i = 32 * it + col;
        const uint64_t mi = shfl_u64(topo.mask, i);
        const float Li = __shfl(L2, i, 64);
        for (int jt = it; jt >= 0; --jt) {
            bf16x8 vf[2];
            const uint32_t ko = (uint32_t)min(32 * jt + col, last) * rq + qoff_half;
            if (jt == it) {
#pragma unroll
                for (int st = 0; st < 2; ++st)
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        vf[st][e] = lv[(16 * st + 8 * (e >> 2) + 4 * half + (e & 3)) * 32 + col];
            } else {
#pragma unroll
                for (int t = 0; t < KS; ++t) kf[t] = load16(ku + (ko + 16 * t));
#pragma unroll
                for (int st = 0; st < 2; ++st)
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        vf[st][e] = vu[(uint32_t)(32 * jt + 16 * st + 8 * (e >> 2) + 4 * half + (e & 3)) * rv + ooff];
            }
            // S^T tile: A = K rows j = 32jt + col, B = Q fragments of tile it
            f32x16 s;
#pragma unroll
            for (int e = 0; e < 16; ++e) s[e] = 0.f;
#pragma unroll
            for (int t = 0; t < KS; ++t) s = mfma32(kf[t], qf[t], s);
            // W^T in accumulator layout: element e pairs node i with
            // j = 32jt + 8(e/4) + 4half + e%4; non-ancestors are selected to 0
            float w[16];
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int j = 32 * jt + 8 * (e >> 2) + 4 * half + (e & 3);
                const bool anc = (mi >> j) & 1ull;
                const float d = __builtin_amdgcn_exp2f(Li - row_val(L2, 32 * jt, e));
                w[e] = anc ? s[e] * d : 0.f;
            }
            // two K-steps of 16 ancestors: element e of step st is w[8st + e], matching vf[st]
#pragma unroll
            for (int st = 0; st < 2; ++st) {
                bf16x8 wh, wl;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    __bf16 xh, xl;
                    split_bf16(w[8 * st + e], xh, xl);
                    wh[e] = xh;
                    wl[e] = xl;
                }
                acc = mfma32(wh, vf[st], acc);
                acc = mfma32(wl, vf[st], acc);
            }
        }
        wait_lds_reads();  // this tile's LDS reads are done: the next tile may refill it

        // ---- output rows i = 32it + 8(e/4) + 4half + e%4 of column c0 + col
        if (n >= 32 * it + 32) {
#pragma unroll
            for (int e = 0; e < 16; ++e)
                ou[(uint32_t)(32 * it + 8 * (e >> 2) + 4 * half + (e & 3)) * rv + ooff] = acc[e];
        } else {
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int ir = 32 * it + 8 * (e >> 2) + 4 * half + (e & 3);
                if (ir < n) ou[(uint32_t)ir * rv + ooff] = acc[e];
            }
        }
    }
}

// Trees of 1..32 nodes (and the status of every tree the big kernel does not take).
// One wavefront per (sequence, head, 64-column group), 16x16 matrix-core tiles:
// lane = (n, g) with n = lane % 16, g = lane / 16; node tiles it/jt = 0, 1 hold nodes
// 16it .. 16it+15.
//
// H_0 term, all v_mfma_f32_16x16x32_bf16. The H_0 slice is loaded straight into
// registers with row-contiguous 16-byte loads: load s = 8t + e gives lane (n, g) row
// 32t + 8g + e, columns 4n .. 4n+3, and one load instruction covers 4 full rows. Over
// the 8 loads of k-step t, lane (n, g) then holds rows 32t + 8g .. +7 of each of its
// columns: exactly the B operand of a 16x16x32 product whose output column n stands
// for state column 4n + c. H_0 never goes through LDS. It is split bf16 hi + lo (two
// products, about 16 mantissa bits); the A operand is the bf16 Q fragment of the same
// k-step, shared with the intra-tree term.
//
// Intra-tree term on bf16 matrix cores (v_mfma_f32_16x16x32_bf16):
//  - S^T tile (jt, it) = K_jt . Q_it^T over d_k; K comes from LDS (DMA, 16-byte pieces
//    XOR-swizzled by row so the fragment reads are conflict-free), Q from registers;
//  - the accumulator layout (lane (n, g) holds j = 16jt + 4g + r for node i = 16it + n)
//    is used in place as the A operand of W.V, with contraction index 8g + e standing
//    for node j = 4g + e (e < 4) or 16 + 4g + e - 4 (e >= 4); V is gathered from LDS in
//    the same order;
//  - W = S * 2^{L_i - L_j} on ancestors, selected to 0 elsewhere, split bf16 hi + lo.
// Both terms land in the same accumulator layout: lane (n, g) holds node 16it + 4g + r,
// state columns 4n .. 4n+3 across its four tiles, stored as one 16-byte write per row.
template <int DK, int DV>
__global__ __launch_bounds__(64) void verify_mfma_tree32_kernel(
    const float *__restrict__ H0, const __bf16 *__restrict__ q, const __bf16 *__restrict__ k,
    const __bf16 *__restrict__ v, const float *__restrict__ gate,
    const int32_t *__restrict__ parent, const int32_t *__restrict__ node_offsets,
    float *__restrict__ out, int32_t *__restrict__ tree_status, int H, int T, int U, int max_n) {
    constexpr int CW = DV < 64 ? DV : 64;   // state columns per wavefront
    constexpr int CPL = CW / 16;            // columns per lane: 4 (2 when d_v = 32)
    constexpr int G = DV / CW;              // column groups per unit
    constexpr int KT = DK / 32;             // k-steps of the bf16 products
    constexpr int HS = DK / 4;              // 16-byte H_0 loads per lane (4 rows each)
    constexpr int PPR = DK / 8;             // 16-byte pieces per K row
    constexpr int VPR = CW / 8;             // 16-byte pieces per V row (of this wave's columns)
    typedef float hvec __attribute__((ext_vector_type(CPL)));
    typedef __bf16 vvec __attribute__((ext_vector_type(CPL)));
    __shared__ bf16x8 s_k[32 * PPR];        // K rows 0..31: piece p of row j at slot j*PPR + (p ^ j%PPR)
    __shared__ __bf16 s_v[32 * CW];         // V rows 0..31 of the wave's columns, row j at [CW j]

    const int lane = lane_id();
    const int n16 = lane & 15, g = lane >> 4;
    int unit, cg;
    if (G == 1) {
        unit = blockIdx.x;
        cg = 0;
    } else {
        const int slot = blockIdx.x >> 3;
        cg = slot % G;
        unit = (slot / G) * 8 + (blockIdx.x & 7);
        if (unit >= U) return;
    }
    const int b = unit / H, h = unit - b * H;
    const int c0 = cg * CW;
    const bool writer = tree_status != nullptr && h == 0 && cg == 0 && lane == 0;

    const TreeRange tr = tree_range(node_offsets, b, T, max_n);
    if (tr.status != BOLE_TREE_OK) {
        if (writer) tree_status[b] = tr.status;
        return;
    }
    if (tr.n > 32) return;  // the big kernel's
    const int lo = tr.lo, n = tr.n;
    if (n == 0) {
        if (writer) tree_status[b] = BOLE_TREE_OK;
        return;
    }
    const int last = n - 1;
    const uint32_t rq = (uint32_t)H * DK, rv = (uint32_t)H * DV;
    const __bf16 *qu = q + (size_t)lo * rq + (size_t)h * DK;
    const __bf16 *ku = k + (size_t)lo * rq + (size_t)h * DK;
    const __bf16 *vu = v + (size_t)lo * rv + (size_t)h * DV + c0;
    float *ou = out + (size_t)lo * rv + (size_t)h * DV + c0;
    const float *hu = H0 + (size_t)unit * DK * DV + c0;

    // ---- 1. issue every load
    const uint32_t node = (uint32_t)min(lane, last);
    const int p_raw = parent[lo + node];
    const float g_raw = gate[(size_t)lo * H + h + node * (uint32_t)H];
    // Q fragments: tile it, k-step t: row 16it + n, elements 32t + 8g .. +7
    bf16x8 qf[2][KT];
#pragma unroll
    for (int it = 0; it < 2; ++it)
#pragma unroll
        for (int t = 0; t < KT; ++t)
            qf[it][t] = load16_stream(qu + ((uint32_t)min(16 * it + n16, last) * rq + 32 * t + 8 * g));
    // K rows -> LDS: instruction s fills slots 64s .. 64s+63, i.e. rows (64/PPR)s ..; lane
    // l fills slot 64s + l = row j, slot-in-row l % PPR, with piece (l % PPR) ^ (j % PPR)
#pragma unroll
    for (int s = 0; s < 32 * PPR / 64; ++s) {
        const int j = (64 / PPR) * s + lane / PPR;
        const int pc = (lane % PPR) ^ (j % PPR);
        dma16_stream(ku + ((uint32_t)min(j, last) * rq + 8 * pc), s_k + 64 * s);
    }
    // V rows -> LDS: lane l of instruction s takes row (64/VPR)s + l/VPR, piece l % VPR
#pragma unroll
    for (int s = 0; s < 32 * VPR / 64; ++s) {
        const int j = (64 / VPR) * s + lane / VPR;
        dma16_stream(vu + ((uint32_t)min(j, last) * rv + 8 * (lane % VPR)), s_v + 512 * s);
    }
    // H_0 slice: step s = 8t + e, lane (n, g): row 32t + 8g + e, columns CPL*n .. +CPL-1
    hvec hreg[HS];
#pragma unroll
    for (int s = 0; s < HS; ++s)
        hreg[s] = __builtin_nontemporal_load(reinterpret_cast<const hvec *>(
            hu + ((uint32_t)(32 * (s >> 3) + 8 * g + (s & 7)) * DV + CPL * n16)));

    // ---- 2. topology and base-2 cumulative decay, lane = node
    const float lg2 = lane < n ? __builtin_amdgcn_logf(g_raw) : 0.f;
    const WaveTopoL topo = wave_topology_cumlog(p_raw, lg2, n);
    if (writer) tree_status[b] = topo.bad;
    if (topo.bad) {
        wait_all_memory();  // no DMA may still target this workgroup's LDS after exit
        for (int i = g; i < n; i += 4)
#pragma unroll
            for (int c = 0; c < CPL; ++c) ou[(uint32_t)i * rv + CPL * n16 + c] = __builtin_nanf("");
        return;
    }
    const float L2 = topo.L;
    float Lrow[2][4];  // L of node 16it + 4g + r (accumulator rows)
#pragma unroll
    for (int it = 0; it < 2; ++it)
#pragma unroll
        for (int r = 0; r < 4; ++r) Lrow[it][r] = __shfl(L2, 16 * it + 4 * g + r, 64);
    float Lcol[2];
    uint64_t mcol[2];  // L and ancestor mask of node 16it + n
#pragma unroll
    for (int it = 0; it < 2; ++it) {
        Lcol[it] = __shfl(L2, 16 * it + n16, 64);
        mcol[it] = shfl_u64(topo.mask, 16 * it + n16);
    }
    wait_all_memory();

    // ---- 3. intra-tree weights: S^T tiles (jt, it) = (0,0), (0,1), (1,1)
    f32x4 st00 = {0.f, 0.f, 0.f, 0.f}, st01 = st00, st11 = st00;
#pragma unroll
    for (int t = 0; t < KT; ++t) {
        const int p = 4 * t + g;
        const bf16x8 k0 = s_k[n16 * PPR + (p ^ (n16 % PPR))];
        const bf16x8 k1 = s_k[(16 + n16) * PPR + (p ^ ((16 + n16) % PPR))];
        st00 = mfma16_bf16(k0, qf[0][t], st00);
        st01 = mfma16_bf16(k0, qf[1][t], st01);
        st11 = mfma16_bf16(k1, qf[1][t], st11);
    }
    // W, as the A operand of W.V for row tile it: element e <-> node j(e) (see above)
    auto weight = [&](float s_val, int it, int jt, int r) {
        const int j = 16 * jt + 4 * g + r;
        const bool anc = (mcol[it] >> j) & 1ull;
        const float d = __builtin_amdgcn_exp2f(Lcol[it] - Lrow[jt][r]);
        return anc ? s_val * d : 0.f;
    };
    bf16x8 wh[2], wl[2];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        __bf16 xh, xl;
        split_bf16(weight(st00[r], 0, 0, r), xh, xl);
        wh[0][r] = xh;
        wl[0][r] = xl;
        wh[0][4 + r] = static_cast<__bf16>(0.f);
        wl[0][4 + r] = static_cast<__bf16>(0.f);
        split_bf16(weight(st01[r], 1, 0, r), xh, xl);
        wh[1][r] = xh;
        wl[1][r] = xl;
        split_bf16(weight(st11[r], 1, 1, r), xh, xl);
        wh[1][4 + r] = xh;
        wl[1][4 + r] = xl;
    }

    // ---- 4. H_0 term: over the 8 steps of k-step t, lane (n, g) holds rows 32t + 8g + e
    // (e = 0..7) of columns CPL*n + c, which is the B operand of a 16x16x32 product for
    // column tile c; A is the Q fragment of the same k-step. H_0 is split bf16 hi + lo.
    f32x4 acc[2][CPL];
#pragma unroll
    for (int it = 0; it < 2; ++it)
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
            for (int it = 0; it < 2; ++it) {
                acc[it][c] = mfma16_bf16(qf[it][t], bh, acc[it][c]);
                acc[it][c] = mfma16_bf16(qf[it][t], bl, acc[it][c]);
            }
        }
    }
#pragma unroll
    for (int it = 0; it < 2; ++it)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float sc = __builtin_amdgcn_exp2f(Lrow[it][r]);
#pragma unroll
            for (int c = 0; c < CPL; ++c) acc[it][c][r] *= sc;
        }

    // ---- 5. intra-tree term: V operand for column tile c: element e = V[j(8g + e)][CPL*n + c]
    bf16x8 vb[CPL];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int j = e < 4 ? 4 * g + e : 12 + 4 * g + e;
        const vvec x = *reinterpret_cast<const vvec *>(s_v + j * CW + CPL * n16);
#pragma unroll
        for (int c = 0; c < CPL; ++c) vb[c][e] = x[c];
    }
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
#pragma unroll
        for (int it = 0; it < 2; ++it) {
            acc[it][c] = mfma16_bf16(wh[it], vb[c], acc[it][c]);
            acc[it][c] = mfma16_bf16(wl[it], vb[c], acc[it][c]);
        }
    }

    // ---- 6. store: node 16it + 4g + r, columns CPL*n .. +CPL-1
#pragma unroll
    for (int it = 0; it < 2; ++it)
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

bool verify_mfma_applies(const bole_dims_t &d, const void *H0, const void *q, const void *k,
                         const void *v, const void *out) {
    if (d.flags & BOLE_FLAG_FORCE_GENERIC) return false;
    if (d.factor_dtype != BOLE_DTYPE_BF16 || d.gate_kind != BOLE_GATE_SCALAR) return false;
    if (d.d_k != 64 && d.d_k != 128) return false;
    if (d.d_v != 32 && d.d_v != 64 && d.d_v != 128 && d.d_v != 256) return false;
    // 16-byte loads of H_0, q, k, v rows and 16-byte stores of out rows
    const uintptr_t a = reinterpret_cast<uintptr_t>(H0) | reinterpret_cast<uintptr_t>(q) |
                        reinterpret_cast<uintptr_t>(k) | reinterpret_cast<uintptr_t>(v) |
                        reinterpret_cast<uintptr_t>(out);
    if (a % 16 != 0) return false;
    // per-tree element offsets (64 rows of one head's rows, and one H_0 slice) are 32-bit
    const uint64_t row_elems = (uint64_t)d.heads * (uint64_t)(d.d_k > d.d_v ? d.d_k : d.d_v);
    if (row_elems * kMaxTree >= (1ull << 31)) return false;
    // work slots (unit x column group, padded to 8) plus two grid strides fit an int
    const uint64_t groups = d.d_v > 64 ? (uint64_t)d.d_v / 64 : 1;
    return ((uint64_t)d.batch * (uint64_t)d.heads + 8) * groups < (1ull << 30);
}

template <int DK, int DV>
static void launch_shape(const float *H0, const __bf16 *q, const __bf16 *k, const __bf16 *v,
                         const float *gate, const int32_t *parent, const int32_t *node_offsets,
                         float *out, const bole_dims_t &d, int32_t *tree_status,
                         hipStream_t stream) {
    const unsigned U = (unsigned)d.batch * (unsigned)d.heads;
    const int max_n = max_tree_nodes(d.flags);
    {
        // trees of <= 32 nodes: one wave per (unit, 64-column group)
        constexpr int G = DV < 64 ? 1 : DV / 64;
        const unsigned grid = G == 1 ? U : ((U + 7) / 8) * 8 * G;
        verify_mfma_tree32_kernel<DK, DV><<<dim3(grid), dim3(64), 0, stream>>>(
            H0, q, k, v, gate, parent, node_offsets, out, tree_status, d.heads, d.total_nodes,
            (int)U, max_n);
    }
    if (max_n > 32) {
        // trees of 33..64 nodes: one wave per (unit, 32-column slice)
        constexpr int NW = (DV < 64 ? DV : 64) / 32;
        constexpr int G = DV / (32 * NW);
        const unsigned grid = G == 1 ? U : ((U + 7) / 8) * 8 * G;
        verify_mfma_big_kernel<DK, DV><<<dim3(grid), dim3(NW * 64), 0, stream>>>(
            H0, q, k, v, gate, parent, node_offsets, out, tree_status, d.heads, d.total_nodes,
            (int)U);
    }
}

template <int DK>
static void launch_dk(const float *H0, const void *q, const void *k, const void *v,
                      const float *gate, const int32_t *parent, const int32_t *node_offsets,
                      float *out, const bole_dims_t &d, int32_t *tree_status, hipStream_t stream) {
    const __bf16 *qb = static_cast<const __bf16 *>(q), *kb = static_cast<const __bf16 *>(k),
                 *vb = static_cast<const __bf16 *>(v);
    switch (d.d_v) {
        case 32: launch_shape<DK, 32>(H0, qb, kb, vb, gate, parent, node_offsets, out, d, tree_status, stream); break;
        case 64: launch_shape<DK, 64>(H0, qb, kb, vb, gate, parent, node_offsets, out, d, tree_status, stream); break;
        case 128: launch_shape<DK, 128>(H0, qb, kb, vb, gate, parent, node_offsets, out, d, tree_status, stream); break;
        case 256: launch_shape<DK, 256>(H0, qb, kb, vb, gate, parent, node_offsets, out, d, tree_status, stream); break;
        default: break;
    }
}

hipError_t launch_verify_mfma(const float *H0, const void *q, const void *k, const void *v,
                              const float *gate, const int32_t *parent,
                              const int32_t *node_offsets, float *out, const bole_dims_t &d,
                              int32_t *tree_status, hipStream_t stream) {
    if (d.d_k == 64)
        launch_dk<64>(H0, q, k, v, gate, parent, node_offsets, out, d, tree_status, stream);
    else
        launch_dk<128>(H0, q, k, v, gate, parent, node_offsets, out, d, tree_status, stream);
    return hipGetLastError();
}

}  // namespace bole
